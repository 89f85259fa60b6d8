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

// Random single-line reads: each 16-lane group reads the first 4 bytes of
// kLineIters pseudo-random 128-byte lines of buf (one request per group and
// read; lines from a 32-bit integer hash of (group, iteration, seed), taken
// modulo the line count, so every address is inside buf).  POL picks the
// load form: 0 plain, 1 non-temporal, 2 relaxed agent-scope atomic, 3
// relaxed system-scope atomic.  What it answers: how many bytes the L2
// fetches from memory for one small read of a line no other read touches --
// the case of a quantized pool's scale read -- and whether a load form
// changes that.
constexpr int kLineIters = 64;

__device__ __forceinline__ uint32_t line_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

template <int POL>
__global__ void __launch_bounds__(256) probe_line_reads_kernel(const float *__restrict__ buf,
                                                               uint32_t nlines, uint32_t seed,
                                                               uint32_t *sink) {
  const uint32_t grp = (blockIdx.x * 256u + threadIdx.x) >> 4;
  float s = 0.f;
#pragma unroll 8
  for (int it = 0; it < kLineIters; ++it) {
    const uint32_t line = line_hash(grp * 977u + static_cast<uint32_t>(it) * 0x9e3779b9u + seed) % nlines;
    const float *ptr = buf + static_cast<uint64_t>(line) * 32u;
    float x;
    if constexpr (POL == 0) x = *ptr;
    else if constexpr (POL == 1) x = __builtin_nontemporal_load(ptr);
    else if constexpr (POL == 2) x = __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else x = __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    s += x;
  }
  uint32_t x = __float_as_uint(s);
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
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

extern "C" int qsa_probe_line_reads(const void *buf, int64_t buf_bytes, int64_t n_reads, int policy,
                                    uint32_t seed, uint32_t *sink, int64_t sink_words,
                                    hipStream_t stream) {
  // one workgroup = 16 groups of 16 lanes, kLineIters reads each
  constexpr int64_t kReadsPerBlock = 16 * kLineIters;
  if (buf == nullptr || sink == nullptr || policy < 0 || policy > 3) return 1;
  if (buf_bytes < 128 || buf_bytes / 128 > 0xFFFFFFFF || (reinterpret_cast<uintptr_t>(buf) & 127)) return 1;
  if (n_reads < kReadsPerBlock || n_reads % kReadsPerBlock != 0) return 1;
  const int64_t blocks = n_reads / kReadsPerBlock;
  if (blocks > sink_words || blocks > 0x7FFFFFFF) return 1;
  const auto *f = static_cast<const float *>(buf);
  const uint32_t nlines = static_cast<uint32_t>(buf_bytes / 128);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (policy) {
    case 0: hipLaunchKernelGGL(probe_line_reads_kernel<0>, grid, block, 0, stream, f, nlines, seed, sink); break;
    case 1: hipLaunchKernelGGL(probe_line_reads_kernel<1>, grid, block, 0, stream, f, nlines, seed, sink); break;
    case 2: hipLaunchKernelGGL(probe_line_reads_kernel<2>, grid, block, 0, stream, f, nlines, seed, sink); break;
    default: hipLaunchKernelGGL(probe_line_reads_kernel<3>, grid, block, 0, stream, f, nlines, seed, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
