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
// Mapping: one wave per (token, kv head); lanes 0..31 handle the K row and
// lanes 32..63 the V row, 8 channels (one 16-byte load) per lane, so the
// absmax of a group of G channels is a butterfly over G/8 lanes.
#include "qsa_internal.h"

namespace qsa {
namespace {

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

template <int FMT>
__global__ void __launch_bounds__(256) qsa_store_kernel(const StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.n * p.hkv) return;
  const int64_t t = row / p.hkv;
  const int h = static_cast<int>(row - t * p.hkv);
  const int64_t slot = p.loc_i64 ? static_cast<const int64_t *>(p.loc)[t]
                                 : static_cast<int64_t>(static_cast<const int32_t *>(p.loc)[t]);
  if (slot < 0 || slot >= p.slots) {
    if (lane == 0) atomicOr(p.err, kErrStoreSlot);
    return;
  }
  const bool is_v = lane >= 32;
  const int l = lane & 31;
  const __bf16 *src = is_v ? p.v + t * p.v_st + h * p.v_sh : p.k + t * p.k_st + h * p.k_sh;
  const uint4 raw = reinterpret_cast<const uint4 *>(src)[l];
  uint8_t *dst = is_v ? p.vp + slot * p.vp_ss + h * p.vp_sh : p.kp + slot * p.kp_ss + h * p.kp_sh;
  if constexpr (FMT == kFmtBF16) {
    reinterpret_cast<uint4 *>(dst)[l] = raw;
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
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
      uint8_t *sd = is_v ? p.vs + slot * p.vs_ss + h * p.vs_sh : p.ks + slot * p.ks_ss + h * p.ks_sh;
      const int gi = l / lpg;
      if (p.scale_f16)
        reinterpret_cast<_Float16 *>(sd)[gi] = static_cast<_Float16>(sc);
      else
        reinterpret_cast<float *>(sd)[gi] = sc;
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (sc > 0.f) ? __fdiv_rn(x[e], sc) : 0.f;
    if constexpr (FMT == kFmtINT4) {
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = static_cast<int>(fminf(fmaxf(__builtin_rintf(y[e]), -7.0f), 7.0f));
        packed |= static_cast<uint32_t>(q + 8) << (4 * e);
      }
      reinterpret_cast<uint32_t *>(dst)[l] = packed;
    } else {
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (FMT == kFmtINT8)
          c[e] = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(__builtin_rintf(y[e]), -127.0f), 127.0f))) & 0xFFu;
        else
          c[e] = e4m3fn_rne(fminf(fmaxf(y[e], -448.0f), 448.0f));
      }
      uint2 out;
      out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      reinterpret_cast<uint2 *>(dst)[l] = out;
    }
  }
}

}  // namespace

hipError_t launch_store(const StoreParams &p, int fmt, hipStream_t stream) {
  const int64_t rows = p.n * p.hkv;
  if (rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
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
