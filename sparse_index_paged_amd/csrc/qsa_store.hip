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
// Mapping: a wave handles one (token, kv head) row of a quantized pool, or
// two consecutive rows for bf16 pools and ring writes
// (store_rows_per_wave).  Lanes 0..31 work on the K row and lanes 32..63 on
// the V row, 8 channels (one 16-byte load) per lane, and all loads of the
// wave's rows are issued before the first row is processed.  The absmax of
// a group of G channels is a butterfly over G/8 lanes.  Codes, scales and
// bf16 rows go to the pools with non-temporal stores.
//
// x / scale must be the correctly rounded fp32 quotient, because the codes
// round it once more.  The quotient is first taken as x * rcp(scale)
// (within 2 ulp of the rounded quotient), and a cheap test shows whether a
// rounding boundary of the code could lie between the two: for int8 / int4
// the residual x - q * scale of the rounded code q (one fused multiply-add),
// for fp8 the hardware e4m3fn conversion of the value moved by +-2^-20 of
// itself (both must give one code).  Only where the test fails is the full
// IEEE division done, so the codes equal those of the division everywhere.
#include "qsa_internal.h"

namespace qsa {
namespace {

// Rows (token, KV head) per wave: one for quantized pools without a ring
// (the most waves in flight); two for bf16 rows and for ring writes.  A
// ring write needs both KV heads of a token in one wave, because the
// token's claim is tested for both before either clears it (rows 2t and
// 2t + 1 share a wave when the count is even).  Every store to a pool is
// non-temporal: the rows are not read back by this launch, and streaming
// them past the L2 measured faster for every format.
template <int FMT>
constexpr int store_rows_per_wave(bool ring) {
  return (FMT == kFmtBF16 || ring) ? 2 : 1;
}

typedef short i16x2 __attribute__((ext_vector_type(2)));

// OCP e4m3fn codes of a and b (|a|, |b| <= 448), rounded to nearest even by
// the gfx950 conversion (scale 1): a in bits 0..7, b in bits 8..15.
__device__ __forceinline__ uint32_t e4m3fn_pair(float a, float b) {
  const i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, a, b, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r) & 0xFFFFu;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// x / sc rounded once (the IEEE quotient), 0 for a zero scale
__device__ __forceinline__ float quotient(float x, float sc) { return sc > 0.f ? __fdiv_rn(x, sc) : 0.f; }

template <int FMT, int kRowsPerWave>
__global__ void __launch_bounds__(256) qsa_store_kernel(const StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * kRowsPerWave;
  const int64_t nrows = p.n * p.hkv;
  const bool is_v = lane >= 32;
  const int l = lane & 31;

  // ---- all loads of the wave's rows first (with a ring, the claims first:
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
      if (ring) {
        claim[i] = p.claim[static_cast<uint32_t>(slot[i]) & p.ring_mask];
      } else {
        const __bf16 *src = is_v ? p.v + t * p.v_st + h * p.v_sh : p.k + t * p.k_st + h * p.k_sh;
        raw[i] = reinterpret_cast<const uint4 *>(src)[l];
      }
    }
  }
  // a ring write reads only the rows of the tokens that hold their claim
  // (one token per ring row): the others' rows are never loaded
  if (ring) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t row = row0 + i;
      if (row < nrows) {
        const int64_t t = (p.hkv == 2) ? (row >> 1) : row;
        const int h = static_cast<int>(row - t * p.hkv);
        if (claim[i] == static_cast<int32_t>(t + 1)) {
          const __bf16 *src = is_v ? p.v + t * p.v_st + h * p.v_sh : p.k + t * p.k_st + h * p.k_sh;
          raw[i] = reinterpret_cast<const uint4 *>(src)[l];
        }
      }
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
      __builtin_nontemporal_store(raw[i].x, reinterpret_cast<uint32_t *>(dst) + 4 * l);
      __builtin_nontemporal_store(raw[i].y, reinterpret_cast<uint32_t *>(dst) + 4 * l + 1);
      __builtin_nontemporal_store(raw[i].z, reinterpret_cast<uint32_t *>(dst) + 4 * l + 2);
      __builtin_nontemporal_store(raw[i].w, reinterpret_cast<uint32_t *>(dst) + 4 * l + 3);
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
          __builtin_nontemporal_store(static_cast<_Float16>(sc), reinterpret_cast<_Float16 *>(sd) + gi);
        else
          __builtin_nontemporal_store(sc, reinterpret_cast<float *>(sd) + gi);
      }
      // Codes from y = x * rcp(sc), within 2 ulp of the IEEE quotient x / sc;
      // only where that could change a code is the quotient itself taken.
      const bool zs = !(sc > 0.f);  // zero scale: zero codes
      const float rs = zs ? 0.f : __builtin_amdgcn_rcpf(sc);
      uint32_t c[8];
      if constexpr (FMT == kFmtFP8) {
        // the codes of y(1 - 2^-20) and y(1 + 2^-20) agree only when no
        // midpoint of the e4m3fn grid (and not the clamp) lies within
        // 2^-20 |y| of y, which holds the quotient; rounding is monotonic
        constexpr float kDown = 1.0f - 0x1p-20f, kUp = 1.0f + 0x1p-20f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float y0 = clamp448(x[e] * rs), y1 = clamp448(x[e + 1] * rs);
          uint32_t two = e4m3fn_pair(clamp448(y0 * kDown), clamp448(y1 * kDown));
          if (two != e4m3fn_pair(clamp448(y0 * kUp), clamp448(y1 * kUp)))
            two = e4m3fn_pair(clamp448(quotient(x[e], sc)), clamp448(quotient(x[e + 1], sc)));
          if (zs) two = 0u;
          c[e] = two & 0xFFu;
          c[e + 1] = two >> 8;
        }
      } else {
        // q = rint(y) is the code's rounding of the IEEE quotient Q' = x / sc
        // when the residual x - q * sc (one fused multiply-add, rounded once)
        // puts the exact quotient within 1/2 - kQ 2^-20 of q: Q' differs from
        // it by at most half an ulp (2^-18 for |Q| < 128, 2^-22 for |Q| < 8),
        // so Q' is no half-integer tie and rounds to q as well (beyond kQ the
        // clamp decides).  Otherwise (or for a non-finite value) Q' is taken.
        const float half = zs ? INFINITY : sc * (0.5f - kQ * 0x1p-20f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float q = __builtin_rintf(x[e] * rs);
          if (!(fabsf(__builtin_fmaf(-q, sc, x[e])) < half)) q = __builtin_rintf(quotient(x[e], sc));
          q = fminf(fmaxf(q, -kQ), kQ);
          if constexpr (FMT == kFmtINT8)
            c[e] = static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu;
          else
            c[e] = static_cast<uint32_t>(static_cast<int>(q) + 8);
        }
      }
      if constexpr (FMT == kFmtINT4) {
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) packed |= c[e] << (4 * e);
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(dst) + l);
      } else {
        uint2 out;
        out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        __builtin_nontemporal_store(out.x, reinterpret_cast<uint32_t *>(dst) + 2 * l);
        __builtin_nontemporal_store(out.y, reinterpret_cast<uint32_t *>(dst) + 2 * l + 1);
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

template <int FMT>
void launch_store_fmt(const StoreParams &p, int64_t rows, hipStream_t stream) {
  const bool ring = p.claim != nullptr;
  const int64_t per_block = 4 * store_rows_per_wave<FMT>(ring);
  const dim3 grid(static_cast<unsigned>((rows + per_block - 1) / per_block));
  if (store_rows_per_wave<FMT>(ring) == 2)
    hipLaunchKernelGGL((qsa_store_kernel<FMT, 2>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((qsa_store_kernel<FMT, 1>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_store(const StoreParams &p, int fmt, hipStream_t stream) {
  const int64_t rows = p.n * p.hkv;
  if (rows <= 0) return hipSuccess;
  switch (fmt) {
    case kFmtBF16: launch_store_fmt<kFmtBF16>(p, rows, stream); break;
    case kFmtFP8: launch_store_fmt<kFmtFP8>(p, rows, stream); break;
    case kFmtINT8: launch_store_fmt<kFmtINT8>(p, rows, stream); break;
    case kFmtINT4: launch_store_fmt<kFmtINT4>(p, rows, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
