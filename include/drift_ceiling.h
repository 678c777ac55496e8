/* Plain-transfer bandwidth of the drift kernels' access patterns, for measurement only.
 *
 * The paired scoring pass reads each active row's logits once and is bound by HBM
 * bandwidth; its rate is compared with the GPU's nominal peak. No kernel reaches that
 * figure, so a benchmark also reports the share of what a plain read of the same bytes,
 * with the same access pattern, reaches on the same GPU; likewise for the gradient pass
 * (dlogits), which reads active rows and writes every row, against a plain copy of the
 * same rows. This library holds those transfers and nothing of the method (no operation
 * of the pages is computed here); it is not part of the drift library.
 *
 * Built as libdrift_ceiling.so beside libdrift.so. Same conventions as drift.h: device
 * pointers, caller-owned memory, stream-ordered, no allocation, no state.
 */
#ifndef DRIFT_CEILING_H
#define DRIFT_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRIFT_CEILING_OK 0
#define DRIFT_CEILING_EINVAL (-1) /* null, misaligned or out-of-range argument */
#define DRIFT_CEILING_EHIP (-2)   /* the launch failed */

/* Number of uint32 words drift_read_ceiling writes to `sink` per row pair. */
#define DRIFT_CEILING_SINK_WORDS 4

/* Reads rows [0, rows) of two row-major arrays `a` and `b` (device memory), row_bytes of
 * each row, rows stride_bytes apart, as the scoring kernels read a row pair: one block of
 * 256 threads per row pair, 16-byte nontemporal loads, eight loads per array in flight per
 * lane. The bytes are folded with XOR and written to sink[DRIFT_CEILING_SINK_WORDS * r + w]
 * (one word per wave) so that no load can be dropped; the values have no meaning.
 *   a, b          device pointers, 16-byte aligned (may be null when rows == 0)
 *   rows          0 <= rows < 2^31
 *   row_bytes     bytes read per row of each array: > 0 and a multiple of 16
 *   stride_bytes  distance between rows: >= row_bytes and a multiple of 16
 *   sink          device, DRIFT_CEILING_SINK_WORDS * rows uint32, 4-byte aligned
 *                 (may be null when rows == 0)
 *   stream        hipStream_t (null = the default stream)
 * Returns DRIFT_CEILING_OK, or an error before anything is launched (EINVAL), or EHIP
 * when the launch fails. Does not synchronize. */
int drift_read_ceiling(const void* a, const void* b, int64_t rows, int64_t row_bytes,
                       int64_t stride_bytes, uint32_t* sink, void* stream);

/* Copies rows [0, rows) of `src` to `dst` (device memory) as the gradient pass moves them:
 * one block of 256 threads per row; a row whose `active` byte is non-zero (every row when
 * `active` is null) is read with 16-byte nontemporal loads, `unroll` loads in flight per
 * lane, and written with 16-byte nontemporal stores; any other row is written as zeros.
 *   src, dst      device pointers, 16-byte aligned (may be null when rows == 0)
 *   rows          0 <= rows < 2^31
 *   row_bytes     bytes per row: > 0 and a multiple of 16
 *   src_stride, dst_stride   distances between rows: >= row_bytes, multiples of 16
 *   active        device uint8 [rows], or null
 *   unroll        4 or 8
 *   stream        hipStream_t (null = the default stream)
 * Returns DRIFT_CEILING_OK, or an error before anything is launched (EINVAL), or EHIP
 * when the launch fails. Does not synchronize. */
int drift_copy_ceiling(const void* src, void* dst, int64_t rows, int64_t row_bytes,
                       int64_t src_stride, int64_t dst_stride, const uint8_t* active,
                       int unroll, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DRIFT_CEILING_H */
