/*
 * qsa_stamps.h -- measurement build libqsa_stamps.so (not part of
 * libqsa.so's decode ABI).
 *
 * libqsa_stamps.so is libqsa.so compiled with per-workgroup phase stamps in
 * the decode kernel; it exports everything qsa.h declares plus the call
 * below.  After qsa_debug_set_phase_stamps(buf, words), every decode launch
 * whose grid has at most words / 8 workgroups makes thread 0 of workgroup
 * i write the device's 100 MHz wall clock (s_memrealtime) into
 * buf[8 i + k] at these points of that workgroup:
 *   k = 0  kernel entry,
 *   k = 1  its row's cu_seqlens entries have arrived,
 *   k = 2  the rows of its first wave's first tile have arrived,
 *   k = 3  its first wave's loop has ended,
 *   k = 4  the workgroup's waves are merged,
 *   k = 5  (split rows) the arrival count is taken,
 *   k = 6  the output is written (unsplit rows, and the last split).
 * Slots a workgroup does not reach keep what the caller put there.  buf is a
 * device pointer owned by the caller (null switches the stamps off); launches
 * with larger grids write none.  The outputs are those of libqsa.so.  Returns 0.
 * The phase breakdown of a decode call (bench.py --mode phases) is read
 * from these stamps.
 */
#ifndef QSA_STAMPS_H_
#define QSA_STAMPS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qsa_debug_set_phase_stamps(void *buf, int64_t words);

#ifdef __cplusplus
}
#endif

#endif /* QSA_STAMPS_H_ */
