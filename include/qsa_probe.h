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

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H_ */
