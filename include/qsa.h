/*
 * qsa.h -- C ABI of the packed QSA (Qwen sparse attention) decode library
 * for AMD Instinct MI355X (gfx950).  Library: libqsa.so.
 *
 * The operation (page "fix(qsa): restore SM121 correctness with Humanize and
 * Kernel Design Agent", section "Changes"): every packed row b holds exactly
 * one bf16 query of Hq heads, head dim 256, with 12 query heads per KV head
 * (24 Q / 2 KV, or 12 Q / 1 KV).  Row b attends over the pool rows listed in
 * sel_indices[cu_seqlens[b] .. cu_seqlens[b+1]) -- at most 2055 entries, read
 * in list order, a repeated slot counted every time it is listed (page
 * "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
 * probes").  For Q head h, with g = h / 12:
 *
 *     s_j    = (q[b,h,:] . K[sel_j, g, :]) / 16
 *     out    = sum_j softmax(s)_j * V[sel_j, g, :]          (bf16, RNE)
 *     lse    = log(sum_j exp(s_j))                           (fp32, natural log)
 *
 * A zero-length row gives out = 0 and lse = -inf.
 *
 * Quantized pools (page "feat(qsa): quantized KV pools with dequant-on-gather
 * (fp8/int8/int4)", part 4 "Modifications") are dequantized while the rows
 * are gathered: element d of a row is code(d) * scale[d / group_size].
 *
 * Conventions for every entry point:
 *   - Pointers inside qsa_tensor are device pointers owned by the caller.
 *     The library never frees them and keeps none of them after returning.
 *   - Strides are in elements of the tensor's dtype (for QSA_DTYPE_U4X2 an
 *     element is one byte holding two codes).  The last dimension must be
 *     contiguous (stride 1), except for lse, which may have any strides.
 *   - Validation is done on the host from shapes/dtypes/strides only; the
 *     host never reads device data.  A failed check returns a status and
 *     sets the thread-local message returned by qsa_last_error().  Nothing
 *     is launched in that case.
 *   - A successful qsa_decode enqueues exactly one kernel on `stream` and
 *     returns without synchronising.
 *   - Errors that only the device can see (a row longer than 2055 or a
 *     cu_seqlens entry outside [0, n_sel], a slot id outside [0, slots))
 *     never fault: the offending row's out/lse are written as NaN and a bit
 *     is set in a sticky device error word (qsa_debug_device_error).
 *   - Workspaces: the library owns the device memory the kernels use beyond
 *     their arguments (split partials, split counters that are zero between
 *     calls, the error word, the indexer's block scores).  Each device has
 *     one shared workspace; qsa_workspace_attach gives a stream a private
 *     one.  A call uses the workspace of its stream: the private one if the
 *     stream has one, else the shared one.  Calls that use the same
 *     workspace must not run concurrently, so concurrent streams each need
 *     a private workspace.  Outside stream capture a workspace is created
 *     or grown on first use; under capture it must already be large enough
 *     (qsa_workspace_reserve / qsa_index_reserve on the capturing stream,
 *     QSA_ERR_WORKSPACE otherwise).  The error word is per workspace.
 *     A workspace never frees memory that a captured graph may still use:
 *     its counters and error word never move, and when its partials or
 *     index scores grow (a larger call, or a larger reservation) the old
 *     buffer is kept until qsa_workspace_detach / qsa_workspace_release.
 *     Graphs captured before a growth therefore replay correctly; graphs
 *     that use a workspace must not be replayed after it is released.
 *     (Page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and
 *     QSA probes", change summary: scratch stays local to the call rather
 *     than shared between callers; here a stream's own workspace is that.)
 */
#ifndef QSA_H_
#define QSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as in the HIP runtime headers. */
typedef struct ihipStream_t *hipStream_t;

#define QSA_ABI_VERSION 5
#define QSA_HEAD_DIM 256
#define QSA_GQA 12
#define QSA_MAX_SEL 2055
#define QSA_MAX_BS 128
#define QSA_INDEX_MAX_TOKENS 262144 /* the indexer's context capacity per row */

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_CONTRACT = 1,  /* a shape / dtype / layout outside the contract   */
  QSA_ERR_ARG = 2,       /* a null pointer or an unknown option             */
  QSA_ERR_WORKSPACE = 3, /* no (or too small a) workspace while capturing   */
  QSA_ERR_HIP = 4        /* a HIP runtime call failed                       */
} qsa_status;

typedef enum qsa_dtype {
  QSA_DTYPE_BF16 = 1,
  QSA_DTYPE_F16 = 2,
  QSA_DTYPE_F32 = 3,
  QSA_DTYPE_I32 = 4,
  QSA_DTYPE_FP8_E4M3FN = 5, /* OCP e4m3fn, one code per byte                  */
  QSA_DTYPE_I8 = 6,         /* signed 8-bit codes                             */
  QSA_DTYPE_U4X2 = 7,       /* two 4-bit codes per byte: channel 2i in the low
                               nibble, 2i+1 in the high nibble, value = nibble-8 */
  QSA_DTYPE_I64 = 8
} qsa_dtype;

/* A strided device tensor of up to 4 dimensions. */
typedef struct qsa_tensor {
  void *data;
  int32_t dtype;       /* qsa_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];   /* in elements */
} qsa_tensor;

/* Scales of a quantized pool pair: k_scale / v_scale are
 * [slots, Hkv, 256 / group_size], both QSA_DTYPE_F32 or both QSA_DTYPE_F16
 * (the pages store fp16 scales).  group_size is 256 (one scale per row), 64
 * or 32 (int4 requires 32 or 64).  Any strides are accepted.  The pages keep
 * the two in separate buffers; a caller that owns the layout may interleave
 * them as views of one [slots, 2, Hkv, 256 / group_size] array (k_scale =
 * [:, 0], v_scale = [:, 1]), so that a slot's K and V scales share one
 * memory line: the same outputs, and a decode that reads one scale line per
 * listed slot instead of two (bs=128 TP1 on MI355X: fp8 54.4 -> 52.2 us,
 * int8 with fp16 scales per 64 channels 58.0 -> 54.3 us). */
typedef struct qsa_kv_scales {
  qsa_tensor k_scale;
  qsa_tensor v_scale;
  int32_t group_size;
} qsa_kv_scales;

/* A tiered pool (page "feat(qsa): quantized KV pools with dequant-on-gather
 * (fp8/int8/int4)", part 4 "Modifications", tiered pool bullet): every
 * token lives as int4 in a full pool and, while it is among the latest
 * written, also as int8 in a ring of R rows (R a power of two).  Ring row
 * r holds the token whose slot id is owner[r]; list entry s reads ring row
 * s & (R-1) when owner[s & (R-1)] == s, otherwise its int4 row.
 *
 *   ring_k, ring_v             [R, Hkv, 256] i8, rows on 16-byte boundaries
 *   ring_k_scale, ring_v_scale [R, Hkv, 4] f16 (one scale per 64 channels)
 *   owner                      [R] i32, contiguous; a row owned by no slot
 *                              holds -1 (any value that is not a listed slot
 *                              id reads the int4 row)
 *   claim                      [R] i32, contiguous, all zero between calls;
 *                              scratch of qsa_kv_store_tiered, which leaves
 *                              it zero (qsa_decode_tiered does not read it)
 *   cold_k, cold_v             [slots, Hkv, 128] u4x2, rows on 16-byte
 *                              boundaries
 *   cold_k_scale, cold_v_scale [slots, Hkv, 8] f16 (one scale per 32 channels)
 * Hkv is 1 or 2 for both tiers.  All memory is owned by the caller. */
typedef struct qsa_tiered_pool {
  qsa_tensor ring_k, ring_v;
  qsa_tensor ring_k_scale, ring_v_scale;
  qsa_tensor owner;
  qsa_tensor claim;
  qsa_tensor cold_k, cold_v;
  qsa_tensor cold_k_scale, cold_v_scale;
} qsa_tiered_pool;

/*
 * qsa_decode -- one packed QSA decode step (one kernel launch).
 *
 *   q           [bs, Hq, 256] bf16.  1 <= bs <= 128; (Hq, Hkv) is (24, 2) or
 *               (12, 1).  Rows must start on 16-byte boundaries.
 *   k_pool      [slots, Hkv, 256] bf16 | fp8_e4m3fn | i8, or
 *               [slots, Hkv, 128] u4x2.  v_pool: same dtype and shape.
 *               Rows must start on 16-byte boundaries.
 *   kv_scales   NULL for bf16 pools, required for quantized pools.
 *   sel_indices [n_sel] int32 slot ids, contiguous.  Only the entries named
 *               by cu_seqlens are read.
 *   cu_seqlens  [bs + 1] int32, contiguous, read on the device only: row b
 *               is sel_indices[cu[b] .. cu[b+1]).  Changing it between graph
 *               replays needs no host involvement.
 *   out         [bs, Hq, 256] bf16, fully overwritten.  Rows must start on
 *               16-byte boundaries.
 *   lse         [bs, Hq] fp32, fully overwritten.
 *   stream      HIP stream the kernel is enqueued on (NULL = default).
 *
 * Uses the split partials, counters and error word of the workspace of
 * `stream` (see the conventions above).
 */
qsa_status qsa_decode(const qsa_tensor *q, const qsa_tensor *k_pool,
                      const qsa_tensor *v_pool, const qsa_kv_scales *kv_scales,
                      const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                      qsa_tensor *out, qsa_tensor *lse, hipStream_t stream);

/*
 * qsa_decode_noalloc -- qsa_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, same contract and the same kernel as
 * qsa_decode; the split partials, split counters and error word live in a
 * fixed scratch array compiled into the library (one per device, 8 MiB of
 * partials), so no call allocates anything, the library's workspaces are
 * never created or used, and the stream needs no reservation.
 *
 *   - A call whose split plan needs more than 8 MiB of partials (only
 *     possible with tuning options that force many splits; the default plan
 *     needs at most 6.2 MB) returns QSA_ERR_WORKSPACE; nothing is launched.
 *   - The first call on a device takes the scratch's device address and
 *     zeroes its counters (one small kernel on `stream`); it must not be
 *     made while `stream` is capturing (QSA_ERR_WORKSPACE).  Later calls,
 *     captured or not, launch exactly one kernel.
 *   - Every call on a device shares that device's scratch: calls that may
 *     overlap in time (different streams without ordering between them)
 *     race on it and must not be made.  Each split counter is zero again
 *     when its launch ends, as with qsa_decode.
 *   - Device-side errors (a row longer than 2055, a bad cu_seqlens entry,
 *     a slot id out of range) give NaN rows as with qsa_decode; their error
 *     bits go to the scratch's own word, which no debug call reads.
 */
qsa_status qsa_decode_noalloc(const qsa_tensor *q, const qsa_tensor *k_pool,
                              const qsa_tensor *v_pool, const qsa_kv_scales *kv_scales,
                              const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                              qsa_tensor *out, qsa_tensor *lse, hipStream_t stream);

/*
 * qsa_kv_store -- quantize new K/V rows and scatter them into the pools
 * (one kernel launch; page "feat(qsa): quantized KV pools with
 * dequant-on-gather (fp8/int8/int4)", part 4 "Modifications": the write is
 * one fused quantize + scatter launch).
 *
 *   k_new, v_new [n, Hkv, 256] bf16, rows on 16-byte boundaries.  n may be 0.
 *   loc          [n] int32 or int64 slot ids, contiguous: row t of k_new /
 *                v_new is written to pool slot loc[t] (all Hkv heads).  The
 *                ids of one call must be distinct; with a repeated id the
 *                slot holds an unspecified mix of the rows written to it
 *                (each scale is one of theirs; codes may mix) and must not
 *                be read until a later call writes it again.  Every other
 *                slot is written exactly.
 *   k_pool, v_pool, kv_scales  as for qsa_decode; written in place.
 *
 * Per (token, KV head, group of group_size channels), in fp32 with ties to
 * even:
 *   i8     scale = absmax / 127, code = clamp(rint(x / scale), -127, 127)
 *   u4x2   scale = absmax / 7,   q = clamp(rint(x / scale), -7, 7), stored
 *          as the nibble q + 8
 *   fp8    scale = absmax / 448, code = e4m3fn(clamp(x / scale, -448, 448))
 *   bf16   the row is copied unchanged (kv_scales must be NULL)
 * An f16 scale is min(scale, 65504) rounded to f16, and the codes are
 * computed from the scale as stored.  A zero scale gives zero codes.
 * Non-finite inputs are outside the contract.
 *
 * A slot id outside [0, slots) skips that token (nothing is written for it)
 * and sets bit 2 of the device error word.  Uses only the error word of
 * the workspace of `stream`: outside capture it is created on first use;
 * under capture it must exist already (QSA_ERR_WORKSPACE otherwise).
 */
qsa_status qsa_kv_store(const qsa_tensor *k_new, const qsa_tensor *v_new,
                        const qsa_tensor *loc, qsa_tensor *k_pool, qsa_tensor *v_pool,
                        const qsa_kv_scales *kv_scales, hipStream_t stream);

/*
 * qsa_decode_tiered -- qsa_decode over a tiered pool (one kernel launch):
 * each listed slot is read from the tier the owner table names, dequantized
 * with that tier's scales.  q, sel_indices, cu_seqlens, out, lse, stream,
 * the workspace and the device error bits are as for qsa_decode; slot ids
 * are checked against the int4 pool's slots.
 */
qsa_status qsa_decode_tiered(const qsa_tensor *q, const qsa_tiered_pool *pool,
                             const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                             qsa_tensor *out, qsa_tensor *lse, hipStream_t stream);

/*
 * qsa_kv_store_tiered -- write new K/V rows into a tiered pool (three
 * kernel launches on `stream`).  k_new, v_new and loc are as for
 * qsa_kv_store (distinct slot ids).  Every token t is quantized to int4
 * with 32-channel scales into slot loc[t] of the int4 pool, and to int8
 * with 64-channel scales into ring row loc[t] & (R-1), whose owner entry
 * becomes loc[t]; the arithmetic is that of qsa_kv_store.  When several
 * tokens of one call map to the same ring row, the one with the largest t
 * is written there.  A slot id outside [0, slots) skips the token and sets
 * bit 2 of the device error word.  pool->claim must be all zero on entry
 * and is all zero again when the launches have run.
 */
qsa_status qsa_kv_store_tiered(const qsa_tensor *k_new, const qsa_tensor *v_new,
                               const qsa_tensor *loc, qsa_tiered_pool *pool, hipStream_t stream);

/*
 * qsa_index -- the indexer step that produces the decode's lists (two
 * kernel launches on `stream`).  The pages name its parts -- MQA scoring,
 * an exact top-k and an index expansion with a fixed 256K-token capacity
 * (page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
 * probes", follow-up "device-planned MQA and QSA quality attribution") --
 * and its row width token_topk + compress_ratio - 1 (page "feat(qsa):
 * quantized KV pools with dequant-on-gather (fp8/int8/int4)", part 4,
 * decode routing paragraph); the rest is this library's reading:
 *
 *   Row b has T_b = context_lens[b] tokens.  Logical block j < n_b =
 *   T_b / c (c = compress_ratio) covers tokens j*c .. j*c + c - 1 and has
 *   one compressed index key, row block_table[b][j] of k_index_pool.  Its
 *   score is s_j = sum_h w_h (q_h . k_j) = qt . k_j over the row's index
 *   heads, with the weighted query qt = sum_h w_h q_h (w_h =
 *   head_weights[b][h], or 1 without weights), in fp32 in this order: per
 *   element d, qt[d] = 0 then qt[d] = fma(w_h, q_h[d], qt[d]) for h = 0, 1,
 *   ...; then s = 0 and s = fma(qt[d], k_j[d], s) for d = 0, 1, ...; -0
 *   reads as +0.
 *   The row keeps the K = budget / c blocks with the largest scores (a tie
 *   goes to the lower block index; every block when n_b <= K), and lists,
 *   in ascending block order, each kept block's c tokens, then the
 *   T_b mod c tokens past the last complete block: min(n_b, K)*c +
 *   T_b mod c entries (at most budget + c - 1), token t written as the KV
 *   slot req_to_token[b][t].  Rows are packed in order into sel_out, and
 *   cu_out receives the offsets (the cu_seqlens of qsa_decode).
 *
 *   q_index       [bs, hi, di] bf16, 1 <= bs <= 128, 1 <= hi <= 64,
 *                 di = 64 or 128, rows on 16-byte boundaries
 *   head_weights  [bs, hi] f32, or NULL
 *   k_index_pool  [n, di] bf16, rows on 16-byte boundaries
 *   block_table   [bs, max_blocks] i32 (max_blocks <= 262144)
 *   req_to_token  [bs, max_tokens] i32 (max_tokens <= 262144)
 *   context_lens  [bs] i32, read on the device only
 *   budget, compress_ratio  1 <= c <= 64, budget a multiple of c,
 *                 budget + c - 1 <= 2055
 *   sel_out       [>= bs * (budget + c - 1)] i32, written
 *   cu_out        [bs + 1] i32, written
 *
 * Uses the score scratch (bs * max_blocks floats) of the workspace of
 * `stream`, created on first use outside stream capture; under capture it
 * must have been reserved with qsa_index_reserve on that stream.  A row whose T_b is negative, above
 * max_tokens or has more blocks than max_blocks lists nothing, and a block
 * table entry outside [0, n) scores -inf; both set bit 3 of the device
 * error word.
 */
qsa_status qsa_index(const qsa_tensor *q_index, const qsa_tensor *head_weights,
                     const qsa_tensor *k_index_pool, const qsa_tensor *block_table,
                     const qsa_tensor *req_to_token, const qsa_tensor *context_lens, int budget,
                     int compress_ratio, qsa_tensor *sel_out, qsa_tensor *cu_out,
                     hipStream_t stream);

/* Create (or grow) the indexer score scratch of the workspace `stream`
 * uses, for calls with up to max_bs rows and max_blocks blocks per row.
 * Call it on the capturing stream before capturing a graph that contains
 * qsa_index. */
qsa_status qsa_index_reserve(int max_bs, int max_blocks, hipStream_t stream);

/* Create (or grow) the workspace `stream` uses for calls with up to max_bs
 * rows and the given head layout, and zero its counters and error word
 * (one small kernel on `stream`).  Call it on the capturing stream before
 * capturing a graph that contains qsa_decode.  Growing keeps the old
 * partials allocated (see the conventions above) and does not
 * synchronise. */
qsa_status qsa_workspace_reserve(int max_bs, int hq, int hkv, hipStream_t stream);

/* Give `stream` a private workspace on the current device, so that its
 * calls can run concurrently with calls on other streams.  It starts empty
 * and is created or grown like the shared one (reserve it before capture).
 * Attaching an attached stream does nothing; at most 64 streams per device
 * (QSA_ERR_WORKSPACE beyond).  Not allowed while `stream` is capturing. */
qsa_status qsa_workspace_attach(hipStream_t stream);

/* Free the private workspace of `stream` (synchronises `stream`, which must
 * still exist); later calls on it use the shared workspace.  A stream
 * without one is left as it is.  Not allowed while `stream` is capturing. */
qsa_status qsa_workspace_detach(hipStream_t stream);

/* Re-zero the split counters and the error word of the workspace `stream`
 * uses (one small kernel on `stream`). */
qsa_status qsa_workspace_reset(hipStream_t stream);

/* Free every workspace, shared and private, of every device and detach all
 * streams (synchronises each device). */
qsa_status qsa_workspace_release(void);

/* Bytes held by the current device's workspaces, shared and private. */
int64_t qsa_workspace_bytes(void);

/* Thread-local message describing the last failed call ("" if none): the
 * descriptive contract error of page "fix(qsa): restore SM121 correctness
 * with Humanize and Kernel Design Agent", section "Changes" (an unsupported
 * call names the field it violates instead of silently running). */
const char *qsa_last_error(void);

/* Split plan qsa_decode uses for (bs, hkv): number of splits per (row, KV
 * head) and the launch's workgroup count over bf16 pools,
 * ceil(bs * hkv / 8) * 8 * splits.  Quantized and tiered pools place every
 * KV head of a row on one XCD and launch ceil(bs / 8) * 8 * hkv * splits
 * workgroups (the same count unless hkv = 2 and bs mod 8 is 1..4).  The plan
 * depends on (bs, hkv) and the options only, never on live lengths. */
qsa_status qsa_plan(int bs, int hkv, int *splits, int *workgroups);

/* Tuning knobs (bench and tests only):
 *   "split_target"   0 (default): splits from a cost model of a launch with
 *                    every list full; > 0: about this many workgroups
 *   "max_splits"     upper bound on splits per (row, KV head) (default 16)
 *   "min_split_keys" fewest list entries a split is given before another
 *                    split is used (default 256)
 *   "waves_per_workgroup" 4 or 8, or 0 (default): 8 for fp8 / int8 / int4
 *                    and tiered pools when the grid has at most one
 *                    workgroup per CU (256), else 4; 4 for bf16 pools
 *   "splits"         0 (default): as above; k >= 1: exactly k splits per
 *                    (row, KV head), at most max_splits
 *   "xcc_lanes"      1 (default): bf16 workgroups take their (row, KV head)
 *                    slot from the XCD they run on (XCC_ID) on a device that
 *                    passed the dispatch check at its first call outside
 *                    capture (8 XCDs, workgroup i of a launch on XCD
 *                    (i + r) % 8); 0: from blockIdx only.  Outputs are
 *                    bitwise the same either way.
 *   "xcc_lanes_active" (read only) the current device's check: -1 not run
 *                    yet, 0 failed (blockIdx placement), 1 passed
 * Changing them affects later launches and later reservations. */
qsa_status qsa_set_option(const char *name, int64_t value);
qsa_status qsa_get_option(const char *name, int64_t *value);

/* Device pointer and count of the split-counter words (uint32, zero
 * between calls) of the workspace `stream` uses, for audits after a launch.
 * The counter of (row b, KV head g) is word (b * Hkv + g) * 32: one counter
 * per 128-byte line, the words between them stay zero.  The
 * counters are the ones of page "fix(qsa): restore SM121 correctness with
 * Humanize and Kernel Design Agent", section "Optimized kernel": the final
 * split of a (row, KV head) resets its counter in the same launch, so every
 * counter reads zero between calls.  The pointer stays valid until the
 * workspace is detached or released. */
qsa_status qsa_debug_counters(const uint32_t **dev_ptr, int *n, hipStream_t stream);

/* Copy the first n split counters of the workspace `stream` uses to host
 * memory (synchronises `stream`). */
qsa_status qsa_debug_read_counters(uint32_t *host, int n, hipStream_t stream);

/* Enqueue one small kernel on `stream` that adds the sum of all split
 * counters of the workspace `stream` uses to *dev_accum (a device uint32).
 * Safe to use between graph replays; *dev_accum stays 0 while every launch
 * leaves its counters at rest. */
qsa_status qsa_debug_audit_counters(uint32_t *dev_accum, hipStream_t stream);

/* Copy the sticky device error word of the workspace `stream` uses to
 * *host_word (synchronises `stream`; 0 when that workspace does not exist
 * yet).
 * Bit 0: a row's cu_seqlens were out of range or longer than 2055.
 * Bit 1: a slot id was outside [0, slots).
 * Bit 2: a qsa_kv_store slot id was outside [0, slots).
 * Bit 3: a qsa_index row's context length or block table entry was out of
 *        range. */
qsa_status qsa_debug_device_error(uint32_t *host_word, hipStream_t stream);

int qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
