// qsa_probe.hip -- measurement helper (libqsa_probe.so, not part of the
// decode library): the bare random-row gather of a decode call, with
// nothing computed on the rows.  For every listed entry and KV head it
// reads the K row and the V row (row_bytes each) exactly as the decode's
// gather does -- 16 bytes per lane, whole rows per wave instruction -- and
// folds them into an XOR that is written once per workgroup, so the loads
// cannot be dropped.  Its rate is the ceiling a gather-bound decode can
// reach on the same pools and lists.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa_probe.h"

namespace {

// Each wave walks its share of the list 16 entries at a time: per KV head
// the 16 K rows and the 16 V rows of those entries are loaded (NI loads
// each per lane), all before the first is consumed.
template <int LPR>  // lanes per row: row_bytes / 16
__global__ void __launch_bounds__(256) probe_gather_kernel(const uint8_t *__restrict__ k,
                                                           const uint8_t *__restrict__ v,
                                                           int64_t ss, int64_t sh, int hkv,
                                                           const int32_t *__restrict__ sel,
                                                           int64_t n_sel, uint32_t slots,
                                                           int64_t per_wave, uint32_t *sink) {
  constexpr int RPI = 64 / LPR;  // rows per wave instruction
  constexpr int NI = 16 / RPI;   // instructions per 16 rows
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t e0 = wave * per_wave;
  int64_t e1 = e0 + per_wave;
  if (e1 > n_sel) e1 = n_sel;
  const int row0 = (lane / LPR) * NI;
  const int64_t chunk = 16 * (lane % LPR);
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int64_t e = e0; e < e1; e += 16) {
    uint32_t slot[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t j = e + row0 + i;
      j = j < e1 ? j : e1 - 1;
      const uint32_t s = static_cast<uint32_t>(sel[j]);
      slot[i] = s < slots ? s : 0u;
    }
    for (int g = 0; g < hkv; ++g) {
      uint4 kr[NI], vr[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t off = static_cast<int64_t>(slot[i]) * ss + g * sh + chunk;
        kr[i] = *reinterpret_cast<const uint4 *>(k + off);
        vr[i] = *reinterpret_cast<const uint4 *>(v + off);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc.x ^= kr[i].x ^ vr[i].x;
        acc.y ^= kr[i].y ^ vr[i].y;
        acc.z ^= kr[i].z ^ vr[i].z;
        acc.w ^= kr[i].w ^ vr[i].w;
      }
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[4];
  if (lane == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" int qsa_probe_gather(const void *k_pool, const void *v_pool, int64_t slot_stride,
                                int64_t head_stride, int hkv, int row_bytes, const int32_t *sel,
                                int64_t n_sel, int64_t slots, int64_t per_wave, uint32_t *sink,
                                int64_t sink_words, hipStream_t stream) {
  if (k_pool == nullptr || v_pool == nullptr || sel == nullptr || sink == nullptr) return 1;
  if (hkv < 1 || hkv > 2 || slots < 1 || slots > 0x7FFFFFFF || n_sel < 1 || per_wave < 16 ||
      per_wave % 16 != 0)
    return 1;
  if ((slot_stride | head_stride) % 16 != 0 || (reinterpret_cast<uintptr_t>(k_pool) & 15) ||
      (reinterpret_cast<uintptr_t>(v_pool) & 15))
    return 1;
  const int64_t waves = (n_sel + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > sink_words || blocks > 0x7FFFFFFF) return 1;
  const auto *k = static_cast<const uint8_t *>(k_pool);
  const auto *v = static_cast<const uint8_t *>(v_pool);
  const uint32_t s32 = static_cast<uint32_t>(slots);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (row_bytes) {
    case 512: hipLaunchKernelGGL(probe_gather_kernel<32>, grid, block, 0, stream, k, v, slot_stride, head_stride, hkv, sel, n_sel, s32, per_wave, sink); break;
    case 256: hipLaunchKernelGGL(probe_gather_kernel<16>, grid, block, 0, stream, k, v, slot_stride, head_stride, hkv, sel, n_sel, s32, per_wave, sink); break;
    case 128: hipLaunchKernelGGL(probe_gather_kernel<8>, grid, block, 0, stream, k, v, slot_stride, head_stride, hkv, sel, n_sel, s32, per_wave, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
