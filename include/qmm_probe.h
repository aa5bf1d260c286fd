/*
 * qmm_probe.h -- C ABI of libqmm_probe: calibration kernels for the roofline
 * figures of the quantized mul_mat library (not part of the method).
 *
 * A kernel's rate is reported against the MI355X datasheet peaks (HBM 8 TB/s,
 * dense int8 MFMA 5.0 POP/s) and against what a minimal kernel measures on the
 * same part (BitBLAS page, "6. 用 profiler 验证瓶颈": confirm the bound by
 * measurement).  Both probes enqueue on `stream` (a hipStream_t, NULL for the
 * legacy default stream), allocate nothing and never synchronize.  They return
 * 0 on success, 1 for a bad argument (nothing enqueued), 2 for a launch error.
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One kernel that reads `bytes` (a multiple of 16) from the device buffer
 * `buf` once with 16-byte loads, `loads_per_thread` (1, 2, 4 or 8) loads per
 * thread issued before any is used, 256 threads per workgroup.  It writes
 * nothing unless the XOR of all it read equals a fixed 128-bit constant, in
 * which case it writes 4 bytes to `sink16` (device, 16-byte aligned).  Pass a
 * zero-filled buffer and nothing is written. */
int qmm_probe_read(const void *buf, size_t bytes, int loads_per_thread, void *sink16, void *stream);

/* Bytes of the device buffer qmm_probe_mfma_i8 writes (one int per thread). */
size_t qmm_probe_mfma_sink_bytes(void);

/* int8 operations one qmm_probe_mfma_i8 launch performs for `iters`. */
double qmm_probe_mfma_ops(int iters);

/* One kernel of 8 wavefronts per SIMD on 256 CUs, each running four
 * independent chains of `iters` v_mfma_i32_32x32x32_i8 instructions on
 * register operands; every thread then writes one int of the chains' state to
 * `sink` (device, at least qmm_probe_mfma_sink_bytes() bytes). */
int qmm_probe_mfma_i8(void *sink, size_t sink_bytes, int iters, int seed, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QMM_PROBE_H */
