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
//   * scores: a workgroup per 128 blocks of a row, one thread per block.
//     The weighted sum over the index heads is taken on the query side
//     first (qt = sum_h w_h q_h, which the heads' shared key makes exact),
//     so a block costs one dot product of its key row with qt: the kernel
//     reads each key row once and is bound by that gather.  The score is
//     evaluated in the order the contract fixes -- qt element by element
//     over the heads in head order, then one fused multiply-add per key
//     element in element order -- so that the top-k decisions are
//     reproducible exactly.
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
constexpr int kSpeculate = 4096; // score kernel: block tables up to this size are read before the lengths

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Tokens a row lists, from its context length alone (0 for a length
// outside the contract).
__device__ __forceinline__ int row_length(const IndexParams &p, int32_t t) {
  if (t < 0 || t > p.max_tokens || t / p.c > p.max_blocks) return 0;
  const int n = t / p.c, k = p.budget / p.c;
  return (n < k ? n : k) * p.c + t % p.c;
}

// A workgroup of 256 threads scores 128 consecutive blocks of one row.
// The contract's score is s_j = qt . k_j with the row's weighted query
// qt = sum_h w_h q_h, in fp32: qt element by element as a fused
// multiply-add chain over the heads in head order, then one fused
// multiply-add per element of k_j in element order.  Every global load is
// issued first: the block-table entries of the key rows a thread stages
// (16-byte pieces, consecutive lanes on one row), then those pieces, its
// share of the row's queries and the head weights.  Queries, weights and
// key rows go to LDS; thread d < DI forms qt[d] (LDS reads in batches of 8
// heads, so the chain waits for LDS once per batch); thread t < 128 then
// runs block j0 + t's chain over its key row against qt (broadcast reads).
template <int DI>
__global__ void __launch_bounds__(256) qsa_index_score_kernel(const IndexParams p) {
  constexpr int kThreads = 256;
  constexpr int kBlocks = 128;           // blocks per workgroup
  constexpr int NC = DI / 8;             // 16-byte pieces of a key row
  constexpr int KP = kBlocks * NC / kThreads;               // key pieces per thread
  constexpr int kPitch = DI * 2 + 16;    // LDS key-row pitch: rows start 16 B apart in the banks
  constexpr int kQPieces = kMaxIndexHeads * NC / kThreads;  // query pieces per thread
  constexpr int kHB = 8;                 // heads per batch of LDS reads in the qt chain
  static_assert(kThreads % NC == 0 && KP * kThreads == kBlocks * NC, "piece mapping");
  const int b = blockIdx.y;
  const int j0 = static_cast<int>(blockIdx.x) * kBlocks;  // < max_blocks (the grid's width)
  const int tid = threadIdx.x;

  __shared__ __attribute__((aligned(16))) unsigned char keys[kBlocks * kPitch];
  __shared__ __attribute__((aligned(16))) uint4 qs[kMaxIndexHeads * NC];  // [64][DI] bf16
  __shared__ __attribute__((aligned(16))) float qt[DI];
  __shared__ float ws[kMaxIndexHeads];

  // With a block table of at most kSpeculate blocks per row, every load is
  // issued before the row's length arrives: the block-table row has
  // max_blocks entries whatever the length, so entries up to max_blocks - 1
  // are read and the blocks past the row's end go unused (at most 32
  // workgroups per row).  Larger tables wait for the length first, so that
  // short rows do not read keys they do not have.
  // Key piece i of this thread: row (i * kThreads + tid) / NC of the
  // workgroup's blocks, 16-byte chunk ch.
  const int32_t t = p.ctx[b];
  if (p.max_blocks > kSpeculate) {
    const bool ok = t >= 0 && t <= p.max_tokens && t / p.c <= p.max_blocks;
    if (j0 >= (ok ? t / p.c : 0)) return;  // uniform
  }
  const int ch = tid % NC;
  int32_t krow[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int j = j0 + (i * kThreads + tid) / NC;
    krow[i] = p.bt[b * p.bt_sb + (j < p.max_blocks ? j : p.max_blocks - 1)];
  }
  uint4 qv[kQPieces];
#pragma unroll
  for (int i = 0; i < kQPieces; ++i) {
    const int pi = i * kThreads + tid;
    const int h = pi / NC;
    qv[i] = make_uint4(0, 0, 0, 0);
    if (h < p.hi) qv[i] = reinterpret_cast<const uint4 *>(p.q + b * p.q_sb + h * p.q_sh)[pi % NC];
  }
  const float wv = (tid < p.hi) ? (p.w ? p.w[b * p.w_sb + tid] : 1.0f) : 0.0f;
  uint4 kv[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int32_t r = krow[i];
    const int64_t rr = (r >= 0 && r < p.n_k) ? r : 0;
    kv[i] = reinterpret_cast<const uint4 *>(p.k + rr * p.k_ss)[ch];
  }
  const bool row_ok = t >= 0 && t <= p.max_tokens && t / p.c <= p.max_blocks;
  const int n = row_ok ? t / p.c : 0;
  if (j0 >= n) return;  // uniform
#pragma unroll
  for (int i = 0; i < kQPieces; ++i) qs[i * kThreads + tid] = qv[i];
  if (tid < kMaxIndexHeads) ws[tid] = wv;
#pragma unroll
  for (int i = 0; i < KP; ++i)
    *reinterpret_cast<uint4 *>(keys + ((i * kThreads + tid) / NC) * kPitch + ch * 16) = kv[i];
  __syncthreads();
  if (tid < DI) {
    const uint16_t *qh = reinterpret_cast<const uint16_t *>(qs) + tid;
    float a = 0.0f;
    for (int h0 = 0; h0 < p.hi; h0 += kHB) {
      float qx[kHB], wx[kHB];
#pragma unroll
      for (int u = 0; u < kHB; ++u) {  // rows past hi hold zeros and weight 0 (read, unused)
        qx[u] = __uint_as_float(static_cast<uint32_t>(qh[(h0 + u) * DI]) << 16);
        wx[u] = ws[h0 + u];
      }
#pragma unroll
      for (int u = 0; u < kHB; ++u)
        if (h0 + u < p.hi) a = __builtin_fmaf(wx[u], qx[u], a);
    }
    qt[tid] = a;
  }
  __syncthreads();

  const int j = j0 + tid;
  if (tid < kBlocks && j < n) {
    const int32_t row = p.bt[b * p.bt_sb + j];
    const bool row_in = row >= 0 && row < p.n_k;
    if (!row_in) atomicOr(p.err, kErrIndexRow);
    const unsigned char *kr = keys + tid * kPitch;
    const float4 *q4 = reinterpret_cast<const float4 *>(qt);
    float sc = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint4 v = *reinterpret_cast<const uint4 *>(kr + i * 16);
      const float4 q0 = q4[2 * i], q1 = q4[2 * i + 1];
      sc = __builtin_fmaf(q0.x, bf_lo(v.x), sc);
      sc = __builtin_fmaf(q0.y, bf_hi(v.x), sc);
      sc = __builtin_fmaf(q0.z, bf_lo(v.y), sc);
      sc = __builtin_fmaf(q0.w, bf_hi(v.y), sc);
      sc = __builtin_fmaf(q1.x, bf_lo(v.z), sc);
      sc = __builtin_fmaf(q1.y, bf_hi(v.z), sc);
      sc = __builtin_fmaf(q1.z, bf_lo(v.w), sc);
      sc = __builtin_fmaf(q1.w, bf_hi(v.w), sc);
    }
    p.scores[static_cast<int64_t>(b) * p.max_blocks + j] = row_in ? sc + 0.0f : -INFINITY;  // -0 -> +0
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
  __shared__ uint32_t hist[2][256];  // double-buffered: pass r counts in hist[r & 1]
  __shared__ int32_t wsum[2][kSelectWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int32_t s_krem;

  // The row's own length, the lengths of the rows before it (one per
  // thread: bs <= 128 <= kSelectThreads) and then its scores are loaded in
  // that order, so that the offset sum below waits for the lengths only
  // while the score loads are still in flight.
  const int32_t t = p.ctx[b];
  const int32_t tprev = p.ctx[tid < b ? tid : b];
  const float *sc = p.scores + static_cast<int64_t>(b) * p.max_blocks;
  constexpr int kRegKeys = KEYS_IN_REGS ? kMaxRegKeys : 1;
  uint32_t keys[kRegKeys];
  if constexpr (KEYS_IN_REGS) {
    // the row's score slots exist up to max_blocks whatever its length:
    // read them before the length arrives (entries past the row's blocks
    // are masked below)
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      const int j = i * kSelectThreads + tid;
      keys[i] = (j < p.max_blocks) ? __float_as_uint(sc[j]) : 0u;  // float bits; keyed below
    }
  }
  int part = tid < b ? row_length(p, tprev) : 0;
  const bool row_ok = t >= 0 && t <= p.max_tokens && t / p.c <= p.max_blocks;
  const int n = row_ok ? t / p.c : 0, k = p.budget / p.c, c = p.c;
  const bool select = n > k;
  if (tid < 256) hist[0][tid] = 0;

  // ---- this row's offset in the packed output
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) wsum[0][wave] = part;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kSelectWaves; ++w) off += wsum[0][w];
  const int len = row_length(p, t);
  if (tid == 0) {
    p.cu[b + 1] = off + len;
    if (b == 0) p.cu[0] = 0;
    if (!row_ok) atomicOr(p.err, kErrIndexRow);
  }
  if (!row_ok) return;  // uniform; the row lists nothing
  int32_t *out = p.sel + off;
  const int32_t *r2t = p.r2t + b * p.r2t_sb;
  if (!select) {  // every block is taken: the row is every token in order
    for (int i = tid; i < t; i += kSelectThreads) out[i] = r2t[i];
    return;
  }
  if constexpr (KEYS_IN_REGS) {
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      const int j = i * kSelectThreads + tid;
      keys[i] = (j < n) ? order_key(__uint_as_float(keys[i])) : 0u;
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

  // ---- radix select of the k-th largest key.  Pass r counts into
  // hist[r & 1] while the other buffer was cleared during pass r - 1's scan
  // (hist[0] before the first pass), so a pass takes two barriers.
  uint32_t prefix = 0, mask = 0;
  int krem = k;  // keys still to take among those matching `prefix` under `mask`
  for (int shift = 24, r = 0; shift >= 0; shift -= 8, ++r) {
    uint32_t *h = hist[r & 1];
    each_chunk([&](int j, uint32_t key) {
      if (j < n && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l (from the top down)
      uint32_t h4[4];
      int c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h4[i] = h[255 - 4 * lane - i];
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
    } else if (tid >= 256 && tid < 512) {
      hist[(r + 1) & 1][tid - 256] = 0;
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
  const dim3 sgrid(static_cast<unsigned>((p.max_blocks + 127) / 128), static_cast<unsigned>(p.bs));
  if (p.max_blocks > 0) {
    if (p.di == 64)
      hipLaunchKernelGGL(qsa_index_score_kernel<64>, sgrid, dim3(256), 0, stream, p);
    else if (p.di == 128)
      hipLaunchKernelGGL(qsa_index_score_kernel<128>, sgrid, dim3(256), 0, stream, p);
    else
      return hipErrorInvalidValue;
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
