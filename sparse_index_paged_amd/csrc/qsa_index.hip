// qsa_index.hip -- the QSA indexer step on gfx950: block scores, exact
// top-k, expansion of the chosen blocks to KV slots.
//
// What it computes is stated in include/qsa.h (qsa_index).  The pages name
// the step's parts -- MQA scoring, an exact top-k and an index expansion,
// with a fixed 256K-token capacity (page "[Kernel][WIP] Integrate native
// FlashInfer SM70 batch GDN and QSA probes", follow-up "device-planned MQA
// and QSA quality attribution") -- and the row width token_topk +
// compress_ratio - 1 (page "feat(qsa): quantized KV pools with
// dequant-on-gather (fp8/int8/int4)", part 4, decode routing paragraph).
//
// Two launches:
//   * scores: a workgroup per 64 blocks of a row.  A lane holds its block's
//     key row in registers; the heads are spread over the waves (8 when
//     the grid has at most one workgroup per CU, else 4), 8 independent
//     dot products per lane at a time, with the queries read
//     from LDS (broadcast).  The score is evaluated in the order the
//     contract fixes -- per head one fused multiply-add per element in
//     element order, then the weighted heads in head order -- so that the
//     top-k decisions are reproducible exactly.
//   * select: one 1024-thread workgroup per row.  Its offset in the packed
//     output depends only on the context lengths, so every workgroup
//     computes its own; an exact radix select (4 passes of 8 bits over
//     order-preserving 32-bit keys, histograms in LDS) finds the K-th
//     largest key, and one pass in ascending block order keeps the blocks
//     above it plus the lowest-indexed blocks equal to it (wave ballots
//     give each thread its rank), expanding each kept block to its c KV
//     slots.  The tokens past the last complete block follow.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int kMaxIndexHeads = 64;
constexpr int kMaxRegKeys = 16;  // keys per thread held in registers by the select kernel

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Tokens a row lists, from its context length alone (0 for a length
// outside the contract).
__device__ __forceinline__ int row_length(const IndexParams &p, int32_t t) {
  if (t < 0 || t > p.max_tokens || t / p.c > p.max_blocks) return 0;
  const int n = t / p.c, k = p.budget / p.c;
  return (n < k ? n : k) * p.c + t % p.c;
}

// A workgroup scores 64 consecutive blocks of one row: lane l of every wave
// takes block 64*blockIdx.x + l, and wave w of W the heads w, w + W, ..., in
// groups of 8 independent dot products (each one a fused multiply-add chain
// in element order).  The row's queries are converted to fp32 once into
// LDS (read back as broadcasts, 4 elements per read), and each key element
// is converted once for 8 heads.  The per-head results meet in LDS, where
// the first wave adds them up in head order.
template <int DI, int W>
__global__ void __launch_bounds__(64 * W) qsa_index_score_kernel(const IndexParams p) {
  constexpr int NC = DI / 8;  // 16-byte chunks of a bf16 row
  constexpr int kScoreThreads = 64 * W;
  constexpr int kWaves = W;
  constexpr int kGroup = 8;   // dot products in flight per lane
  const int b = blockIdx.y;
  const int32_t t = p.ctx[b];
  const bool row_ok = t >= 0 && t <= p.max_tokens && t / p.c <= p.max_blocks;
  const int n = row_ok ? t / p.c : 0;
  if (static_cast<int>(blockIdx.x) * 64 >= n) return;  // uniform

  __shared__ float4 qf[kMaxIndexHeads * DI / 4];   // [hi][DI] fp32
  __shared__ float dots[kMaxIndexHeads][64];
  for (int i = threadIdx.x; i < p.hi * NC; i += kScoreThreads) {
    const int h = i / NC, c8 = i - h * NC;
    const uint4 v = reinterpret_cast<const uint4 *>(p.q + b * p.q_sb + h * p.q_sh)[c8];
    qf[2 * i] = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
    qf[2 * i + 1] = make_float4(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int j = blockIdx.x * 64 + lane;
  const bool live = j < n;
  const int32_t row = live ? p.bt[b * p.bt_sb + j] : 0;
  const bool row_in = row >= 0 && row < p.n_k;
  if (live && !row_in && wave == 0) atomicOr(p.err, kErrIndexRow);
  uint4 kr[NC];
  const uint4 *kp = reinterpret_cast<const uint4 *>(p.k + static_cast<int64_t>(row_in ? row : 0) * p.k_ss);
#pragma unroll
  for (int i = 0; i < NC; ++i) kr[i] = kp[i];

  for (int h0 = wave; h0 < p.hi; h0 += kWaves * kGroup) {
    float a[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) a[u] = 0.0f;
    // heads h0, h0 + 4, ..., (those < hi)
    const int nh = min(kGroup, (p.hi - h0 + kWaves - 1) / kWaves);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const float kf[8] = {bf_lo(kr[i].x), bf_hi(kr[i].x), bf_lo(kr[i].y), bf_hi(kr[i].y),
                           bf_lo(kr[i].z), bf_hi(kr[i].z), bf_lo(kr[i].w), bf_hi(kr[i].w)};
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        if (u < nh) {
          const float4 q0 = qf[((h0 + kWaves * u) * DI) / 4 + 2 * i];
          const float4 q1 = qf[((h0 + kWaves * u) * DI) / 4 + 2 * i + 1];
          a[u] = __builtin_fmaf(q0.x, kf[0], a[u]);
          a[u] = __builtin_fmaf(q0.y, kf[1], a[u]);
          a[u] = __builtin_fmaf(q0.z, kf[2], a[u]);
          a[u] = __builtin_fmaf(q0.w, kf[3], a[u]);
          a[u] = __builtin_fmaf(q1.x, kf[4], a[u]);
          a[u] = __builtin_fmaf(q1.y, kf[5], a[u]);
          a[u] = __builtin_fmaf(q1.z, kf[6], a[u]);
          a[u] = __builtin_fmaf(q1.w, kf[7], a[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (u < nh) dots[h0 + kWaves * u][lane] = a[u];
  }
  __syncthreads();
  if (wave == 0 && live) {
    float s = 0.0f;
    for (int h = 0; h < p.hi; ++h) {
      const float wh = p.w ? p.w[b * p.w_sb + h] : 1.0f;
      s = __builtin_fmaf(wh, dots[h][lane], s);
    }
    p.scores[static_cast<int64_t>(b) * p.max_blocks + j] = row_in ? s + 0.0f : -INFINITY;  // -0 -> +0
  }
}

// Order-preserving 32-bit key of a float (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of m below this lane.
__device__ __forceinline__ int bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// KEYS_IN_REGS: the row's keys (at most 16 per thread, 16,384 blocks) are
// loaded once into registers for all passes; otherwise every pass reads the
// scores again.
template <bool KEYS_IN_REGS>
__global__ void __launch_bounds__(kSelectThreads) qsa_index_select_kernel(const IndexParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ uint32_t hist[256];
  __shared__ int32_t wsum[2][kSelectWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int32_t s_krem;

  // ---- this row's offset in the packed output
  int part = 0;
  for (int i = tid; i < b; i += kSelectThreads) part += row_length(p, p.ctx[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) wsum[0][wave] = part;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kSelectWaves; ++w) off += wsum[0][w];
  const int32_t t = p.ctx[b];
  const bool row_ok = t >= 0 && t <= p.max_tokens && t / p.c <= p.max_blocks;
  const int len = row_length(p, t);
  if (tid == 0) {
    p.cu[b + 1] = off + len;
    if (b == 0) p.cu[0] = 0;
    if (!row_ok) atomicOr(p.err, kErrIndexRow);
  }
  if (!row_ok) return;  // uniform; the row lists nothing
  const int n = t / p.c, k = p.budget / p.c, c = p.c;
  int32_t *out = p.sel + off;
  const int32_t *r2t = p.r2t + b * p.r2t_sb;
  if (n <= k) {  // every block is taken: the row is every token in order
    for (int i = tid; i < t; i += kSelectThreads) out[i] = r2t[i];
    return;
  }
  const float *sc = p.scores + static_cast<int64_t>(b) * p.max_blocks;
  constexpr int kRegKeys = KEYS_IN_REGS ? kMaxRegKeys : 1;
  uint32_t keys[kRegKeys];
  if constexpr (KEYS_IN_REGS) {
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      const int j = i * kSelectThreads + tid;
      keys[i] = (j < n) ? order_key(sc[j]) : 0u;
    }
  }
  const int nchunk = (n + kSelectThreads - 1) / kSelectThreads;
  // body(j, key) for this thread's block j = i * kSelectThreads + tid of
  // every chunk i < nchunk in order (key 0 when j >= n)
  auto each_chunk = [&](auto &&body) {
    if constexpr (KEYS_IN_REGS) {
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i) {
        if (i >= nchunk) break;  // uniform
        body(i * kSelectThreads + tid, keys[i]);
      }
    } else {
      for (int i = 0; i < nchunk; ++i) {
        const int j = i * kSelectThreads + tid;
        body(j, j < n ? order_key(sc[j]) : 0u);
      }
    }
  };

  // ---- radix select of the k-th largest key
  uint32_t prefix = 0, mask = 0;
  int krem = k;  // keys still to take among those matching `prefix` under `mask`
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    each_chunk([&](int j, uint32_t key) {
      if (j < n && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l (from the top down)
      uint32_t h4[4];
      int c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h4[i] = hist[255 - 4 * lane - i];
        c4 += static_cast<int>(h4[i]);
      }
      int incl = c4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const int excl = incl - c4;
      if (excl < krem && krem <= incl) {
        int run = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run + static_cast<int>(h4[i]) >= krem) {
            s_prefix = prefix | (static_cast<uint32_t>(255 - 4 * lane - i) << shift);
            s_krem = krem - run;
            break;
          }
          run += static_cast<int>(h4[i]);
        }
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 0xFFu << shift;
  }
  const uint32_t thr = prefix;  // the k-th largest key
  const int need_eq = krem;     // keys equal to thr that are taken (the lowest-indexed ones)

  // ---- keep, in ascending block order, the blocks above thr and the
  // first need_eq blocks equal to it; block of rank r fills out[r*c ..]
  int gt_run = 0, eq_run = 0;
  each_chunk([&](int j, uint32_t key) {
    const bool gt = j < n && key > thr;
    const bool eq = j < n && key == thr;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    if (lane == 0) {
      wsum[0][wave] = __popcll(bgt);
      wsum[1][wave] = __popcll(beq);
    }
    __syncthreads();
    int gt_before = gt_run + bits_below(bgt), eq_before = eq_run + bits_below(beq);
    int gt_all = 0, eq_all = 0;
#pragma unroll
    for (int w = 0; w < kSelectWaves; ++w) {
      if (w < wave) {
        gt_before += wsum[0][w];
        eq_before += wsum[1][w];
      }
      gt_all += wsum[0][w];
      eq_all += wsum[1][w];
    }
    if (gt || (eq && eq_before < need_eq)) {
      const int rank = gt_before + (eq_before < need_eq ? eq_before : need_eq);
      if (rank < k)  // always true (k keys are kept); keeps every write inside the row
        for (int e = 0; e < c; ++e) out[rank * c + e] = r2t[j * c + e];
    }
    gt_run += gt_all;
    eq_run += eq_all;
    __syncthreads();
  });
  // ---- the tokens past the last complete block
  for (int i = tid; i < t - n * c; i += kSelectThreads) out[k * c + i] = r2t[n * c + i];
}

}  // namespace

hipError_t launch_index(const IndexParams &p, hipStream_t stream) {
  const dim3 sgrid(static_cast<unsigned>((p.max_blocks + 63) / 64), static_cast<unsigned>(p.bs));
  // with at most one workgroup per CU the waves' LDS-latency-bound chains
  // are the time, so 8 waves (8 heads each) halve them; larger grids keep
  // 4 waves (16 heads each), which were faster there (MI355X, 8K-token rows,
  // 64 heads of dim 128: 4 / 8 rows 34.2 / 34.9 -> 25.7 / 26.3 us; 32 rows
  // 56.4 us with 4 waves against 64.7 with 8)
  // (full 64-block columns only: the grid's last column is often empty and
  // its workgroups return at once)
  // (64-dim heads hold half the key registers, so their 8-wave instance
  // keeps more waves resident and stays ahead up to two workgroups per CU:
  // 16 rows of dim 64, 26.0 -> 23.0 us)
  const bool eight = static_cast<int64_t>(p.max_blocks / 64) * p.bs <= (p.di == 64 ? 512 : 256);
  if (p.max_blocks > 0) {
    switch (p.di * 2 + (eight ? 1 : 0)) {
      case 64 * 2: hipLaunchKernelGGL((qsa_index_score_kernel<64, 4>), sgrid, dim3(256), 0, stream, p); break;
      case 64 * 2 + 1: hipLaunchKernelGGL((qsa_index_score_kernel<64, 8>), sgrid, dim3(512), 0, stream, p); break;
      case 128 * 2: hipLaunchKernelGGL((qsa_index_score_kernel<128, 4>), sgrid, dim3(256), 0, stream, p); break;
      case 128 * 2 + 1: hipLaunchKernelGGL((qsa_index_score_kernel<128, 8>), sgrid, dim3(512), 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (p.max_blocks <= kMaxRegKeys * kSelectThreads)
    hipLaunchKernelGGL(qsa_index_select_kernel<true>, dim3(static_cast<unsigned>(p.bs)), dim3(kSelectThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(qsa_index_select_kernel<false>, dim3(static_cast<unsigned>(p.bs)), dim3(kSelectThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace qsa
