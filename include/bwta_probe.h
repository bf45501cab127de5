/*
 * bwta_probe.h - C ABI of libbwta_probe.so: the two measurement kernels the
 * benchmark uses to measure the ceilings of the MI355X it runs on, so that
 * each kernel's roofline fraction can be stated against the measured figure
 * as well as the datasheet one.  They compute nothing of the method (the
 * binary x ternary product of the BWTA page is in libbwta.so); they exist to
 * be timed.
 *
 * Both take device pointers owned by the caller, enqueue one kernel on
 * `stream` (a hipStream_t; NULL = the default stream), do not synchronize,
 * and return 0, -1 for invalid arguments or -2 for a failed launch.
 */
#ifndef BWTA_PROBE_H_
#define BWTA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` (16-byte aligned, bytes a multiple of 16) once
 * with 16-byte non-temporal loads spread over the whole chip (each wave of a
 * 256-thread block reads 8 consecutive KiB at a time, all loads in flight at
 * once), and store one 32-bit XOR of what each block read to sink[block]
 * (sink: blocks words, blocks <= 8192; blocks = 0 picks one round per wave, at
 * most 8192 blocks).  Timing it gives the read-only HBM bandwidth of a stream of
 * that size. */
int bwta_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                           void* stream);

/* Run `iters` rounds of 16 independent matrix-core products per wave on
 * `waves` waves (one block of 4 waves per compute unit at waves = 1024):
 * fmt 0 = v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 (e2m1) operands (131072
 * operations each), fmt 1 = v_mfma_i32_32x32x32_i8 (65536 operations each).
 * Each wave stores one word of its accumulators to sink[wave] (sink: waves
 * words).  Operations per launch = waves * iters * 16 * (per-product count). */
int bwta_probe_mfma(int fmt, int waves, int iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BWTA_PROBE_H_ */
