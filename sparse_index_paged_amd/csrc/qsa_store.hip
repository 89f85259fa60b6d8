// qsa_store.hip -- fused quantize + scatter of new K/V rows into the pools
// (gfx950).
//
// Page "feat(qsa): quantized KV pools with dequant-on-gather
// (fp8/int8/int4)", part 4 "Modifications": writing a quantized pool is one
// fused quantize + scatter launch.  Per (token, kv head, channel group):
//   int8  scale = absmax / 127, code = clamp(rint(x / scale), -127, 127)
//   int4  scale = absmax / 7,   q = clamp(rint(x / scale), -7, 7), stored as
//         the nibble q + 8, even channel in the low nibble
//   fp8   scale = absmax / 448, code = e4m3fn(clamp(x / scale, -448, 448))
//         (the saturation of the fp8 write path of part 2, which avoids the
//         NaN the cast gives beyond +-448)
// with fp32 arithmetic, ties to even, a zero scale giving zero codes, and
// fp16 scales clamped to 65504 before rounding (the write-kernel bullet of
// the same section); codes are computed from the scale as stored.  bf16
// pools take the rows unchanged.
//
// Tiered pools (same section, tiered pool bullet) are written by three
// launches: the int4 store into the full pool, a claim pass that records
// for every ring row the last token of the call that maps to it, and the
// int8 store into the ring, where only that token writes the row, stamps
// the owner table and clears its claim (so the claim table is zero again
// when the call ends).
//
// Mapping: a wave handles 4 consecutive (token, kv head) rows; lanes 0..31
// work on the K rows and lanes 32..63 on the V rows, 8 channels (one
// 16-byte load) per lane, and all loads of the 4 rows are issued before the
// first row is processed.  The absmax of a group of G channels is a
// butterfly over G/8 lanes.
//
// x / scale must be the correctly rounded fp32 quotient, because the codes
// round it once more.  The quotient is first taken as x * rcp(scale)
// (within 2 ulp of the rounded quotient); only when that value lies within
// 8 ulp of a rounding boundary of the code (a half-integer for int8 / int4,
// a midpoint of the e4m3fn grid for fp8) is the full IEEE division done, so
// the codes equal those of the division everywhere.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kRowsPerWave = 4;

// e4m3fn code of y with |y| <= 448, rounded to nearest even.  Normal codes
// come from rounding the fp32 significand to 3 bits (a carry moves into the
// exponent); below 2^-6 the code is the subnormal multiple of 2^-9.
__device__ __forceinline__ uint32_t e4m3fn_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const float af = __uint_as_float(a);
  uint32_t code;
  if (af < 0x1p-6f)
    code = static_cast<uint32_t>(__builtin_rintf(af * 512.0f));
  else
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | code;
}

// True when rint(v) could change if v moved by up to 8 ulp (or v is not finite).
__device__ __forceinline__ bool near_half_integer(float v) {
  const float d = fabsf(v - floorf(v) - 0.5f);
  return !(d > fmaxf(fabsf(v), 1.0f) * 0x1p-20f);
}

// Same for the e4m3fn rounding of clamp(v, -448, 448).
__device__ __forceinline__ bool near_e4m3_boundary(float v) {
  const float a = fabsf(v);
  if (!(a <= 448.0f)) return !(a > 448.0f) || a < 456.0f;  // NaN, or just above the clamp
  if (a < 0x1p-6f) return near_half_integer(a * 512.0f);
  const int32_t m = static_cast<int32_t>(__float_as_uint(a) & 0xFFFFFu) - 0x80000;
  return m >= -8 && m <= 8;
}

template <int FMT>
__device__ __forceinline__ uint32_t code_of(float y) {
  if constexpr (FMT == kFmtINT8)
    return static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f))) & 0xFFu;
  else if constexpr (FMT == kFmtINT4)
    return static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(__builtin_rintf(y), -7.0f), 7.0f)) + 8);
  else
    return e4m3fn_rne(fminf(fmaxf(y, -448.0f), 448.0f));
}

template <int FMT>
__global__ void __launch_bounds__(256) qsa_store_kernel(const StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * kRowsPerWave;
  const int64_t nrows = p.n * p.hkv;
  const bool is_v = lane >= 32;
  const int l = lane & 31;

  // ---- all loads of the wave's rows first (with a ring, also the claims:
  // every claim this wave tests is read before it clears any)
  uint4 raw[kRowsPerWave];
  int64_t slot[kRowsPerWave];
  int32_t claim[kRowsPerWave];
  const bool ring = p.claim != nullptr;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t row = row0 + i;
    if (row < nrows) {
      const int64_t t = (p.hkv == 2) ? (row >> 1) : row;
      const int h = static_cast<int>(row - t * p.hkv);
      slot[i] = p.loc_i64 ? static_cast<const int64_t *>(p.loc)[t]
                          : static_cast<int64_t>(static_cast<const int32_t *>(p.loc)[t]);
      const __bf16 *src = is_v ? p.v + t * p.v_st + h * p.v_sh : p.k + t * p.k_st + h * p.k_sh;
      raw[i] = reinterpret_cast<const uint4 *>(src)[l];
      if (ring) claim[i] = p.claim[static_cast<uint32_t>(slot[i]) & p.ring_mask];
    }
  }

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t row = row0 + i;
    if (row >= nrows) break;
    const int64_t t = (p.hkv == 2) ? (row >> 1) : row;
    const int h = static_cast<int>(row - t * p.hkv);
    int64_t s = slot[i];
    if (s < 0 || s >= p.slots) {
      if (lane == 0) atomicOr(p.err, kErrStoreSlot);
      continue;
    }
    if (ring) {
      // only the last token of the call that maps to this ring row writes it
      if (claim[i] != static_cast<int32_t>(t + 1)) continue;
      const int64_t r = static_cast<int64_t>(static_cast<uint32_t>(s) & p.ring_mask);
      if (h == p.hkv - 1 && lane == 0) {
        p.owner[r] = static_cast<int32_t>(s);
        p.claim[r] = 0;
      }
      s = r;
    }
    uint8_t *dst = is_v ? p.vp + s * p.vp_ss + h * p.vp_sh : p.kp + s * p.kp_ss + h * p.kp_sh;
    if constexpr (FMT == kFmtBF16) {
      reinterpret_cast<uint4 *>(dst)[l] = raw[i];
    } else {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
      const int lpg = p.group >> 3;  // lanes per scale group
      for (int m = 1; m < lpg; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
      constexpr float kQ = (FMT == kFmtINT8) ? 127.0f : (FMT == kFmtINT4) ? 7.0f : 448.0f;
      float sc = __fdiv_rn(am, kQ);
      if (p.scale_f16) sc = static_cast<float>(static_cast<_Float16>(fminf(sc, 65504.0f)));
      if ((l & (lpg - 1)) == 0) {
        uint8_t *sd = is_v ? p.vs + s * p.vs_ss + h * p.vs_sh : p.ks + s * p.ks_ss + h * p.ks_sh;
        const int gi = l / lpg;
        if (p.scale_f16)
          reinterpret_cast<_Float16 *>(sd)[gi] = static_cast<_Float16>(sc);
        else
          reinterpret_cast<float *>(sd)[gi] = sc;
      }
      const float rs = __builtin_amdgcn_rcpf(sc);
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = x[e] * rs;
        const bool near = (FMT == kFmtFP8) ? near_e4m3_boundary(y) : near_half_integer(y);
        if (near) y = __fdiv_rn(x[e], sc);
        if (!(sc > 0.f)) y = 0.f;
        c[e] = code_of<FMT>(y);
      }
      if constexpr (FMT == kFmtINT4) {
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) packed |= c[e] << (4 * e);
        reinterpret_cast<uint32_t *>(dst)[l] = packed;
      } else {
        uint2 out;
        out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        reinterpret_cast<uint2 *>(dst)[l] = out;
      }
    }
  }
}

__global__ void __launch_bounds__(256) qsa_claim_kernel(const StoreParams p) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= p.n) return;
  const int64_t s = p.loc_i64 ? static_cast<const int64_t *>(p.loc)[t]
                              : static_cast<int64_t>(static_cast<const int32_t *>(p.loc)[t]);
  if (s < 0 || s >= p.slots) return;
  atomicMax(p.claim + (static_cast<uint32_t>(s) & p.ring_mask), static_cast<int32_t>(t + 1));
}

}  // namespace

hipError_t launch_claim(const StoreParams &p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.n + 255) / 256));
  hipLaunchKernelGGL(qsa_claim_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_store(const StoreParams &p, int fmt, hipStream_t stream) {
  const int64_t rows = p.n * p.hkv;
  if (rows <= 0) return hipSuccess;
  const int64_t per_block = 4 * kRowsPerWave;
  const dim3 grid(static_cast<unsigned>((rows + per_block - 1) / per_block));
  switch (fmt) {
    case kFmtBF16: hipLaunchKernelGGL(qsa_store_kernel<kFmtBF16>, grid, dim3(256), 0, stream, p); break;
    case kFmtFP8: hipLaunchKernelGGL(qsa_store_kernel<kFmtFP8>, grid, dim3(256), 0, stream, p); break;
    case kFmtINT8: hipLaunchKernelGGL(qsa_store_kernel<kFmtINT8>, grid, dim3(256), 0, stream, p); break;
    case kFmtINT4: hipLaunchKernelGGL(qsa_store_kernel<kFmtINT4>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
