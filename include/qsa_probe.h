/*
 * qsa_probe.h -- measurement helper library libqsa_probe.so (not part of
 * libqsa.so's decode ABI).
 *
 * qsa_probe_gather reads, for every entry of sel[0 .. n_sel) and every KV
 * head g < hkv, the K row and the V row of that slot -- row_bytes bytes
 * each (512, 256 or 128), at k_pool / v_pool + slot * slot_stride +
 * g * head_stride (byte strides, 16-byte aligned) -- with the same
 * 16-bytes-per-lane whole-row loads as the decode's gather, and nothing
 * else: the bare gather whose rate bounds a gather-bound decode (page "fix(qsa):
 * restore SM121 correctness with Humanize and Kernel Design Agent",
 * section "Optimized kernel": each gathered K/V row is read once for the
 * 12 query heads that share it).  Each wave takes per_wave consecutive
 * entries (a multiple of 16); workgroup i writes the XOR of everything it
 * read to sink[i] (sink_words must cover ceil(ceil(n_sel / per_wave) / 4)
 * workgroups).  Slot ids outside [0, slots) read slot 0.  One kernel launch
 * on `stream`; returns 0, 1 for bad arguments (nothing launched), 2 when
 * the launch failed.
 *
 * qsa_probe_line_reads makes n_reads reads of 4 bytes, each of the first
 * word of a pseudo-random 128-byte line of buf[0 .. buf_bytes) (buf
 * 128-byte aligned, at most 2^32 lines), one request per 16-lane group
 * and read, under one load form: policy 0 plain, 1 non-temporal, 2 relaxed
 * agent-scope atomic, 3 relaxed system-scope atomic.  It stands for the
 * scale reads of a quantized pool (page "feat(qsa): quantized KV pools
 * with dequant-on-gather (fp8/int8/int4)", part 4: a slot's scales live in
 * arrays of their own, so each listed slot's scale is a small read of a
 * line the row read does not touch).  n_reads must be a positive multiple
 * of 1024 (one workgroup per 1024 reads); workgroup i writes a fold of
 * what it read to sink[i] (sink_words >= n_reads / 1024).  seed varies the
 * lines.  One kernel launch on `stream`; returns 0, 1 for bad arguments
 * (nothing launched), 2 when the launch failed.
 */
#ifndef QSA_PROBE_H_
#define QSA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

int qsa_probe_gather(const void *k_pool, const void *v_pool, int64_t slot_stride,
                     int64_t head_stride, int hkv, int row_bytes, const int32_t *sel,
                     int64_t n_sel, int64_t slots, int64_t per_wave, uint32_t *sink,
                     int64_t sink_words, hipStream_t stream);

int qsa_probe_line_reads(const void *buf, int64_t buf_bytes, int64_t n_reads, int policy,
                         uint32_t seed, uint32_t *sink, int64_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H_ */
