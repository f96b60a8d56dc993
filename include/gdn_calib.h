/* gdn_calib.h -- calibration kernels exported by libgdn.so.
 *
 * Two plain kernels that measure what this GPU actually sustains, so that a
 * kernel's roofline fraction can be stated against an achieved peak as well
 * as the published one:
 *
 *   gdn_calib_copy       a streaming device-to-device copy (HBM bandwidth:
 *                        every byte read once and written once);
 *   gdn_calib_mfma_loop  dense bf16 matrix-core work with no memory traffic
 *                        (v_mfma_f32_16x16x32_bf16 or v_mfma_f32_32x32x16_bf16
 *                        on register operands).
 *
 * Neither is part of the gated-delta-rule computation.  Conventions are those
 * of gdn.h: device pointers, the caller's stream (NULL = the null stream), no
 * allocation, no synchronisation; a rejected call enqueues nothing.
 */
#ifndef GDN_CALIB_H
#define GDN_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` bytes from src to dst (device memory, both 16-byte aligned,
 * not overlapping; bytes a multiple of 16).  Workgroups of 256 threads, one
 * tile of 256 * U 16-byte elements each, one pass of the grid; every thread
 * issues its U loads before its first store.  variant selects the form:
 *   0  U = 1 (the fastest form measured on MI355X: 6.1 TB/s over 2 GiB);
 *   1  U = 4;
 *   2  U = 2 with non-temporal loads and stores.
 * Errors: GDN_ERR_NULL_POINTER (src or dst NULL with bytes > 0),
 * GDN_ERR_MISALIGNED, GDN_ERR_BAD_SHAPE (bytes % 16, or the ranges overlap),
 * GDN_ERR_UNSUPPORTED (variant), GDN_ERR_HIP. */
gdn_status gdn_calib_copy(const void* src, void* dst, size_t bytes, int32_t variant,
                          void* hip_stream);

/* Run `workgroups` workgroups of 256 threads (4 waves); every wave issues
 * iters x 8 matrix-core instructions and stores one float (the sum of its
 * accumulators) to out[4 * wg + wave] (out: workgroups * 4 floats, device
 * memory, 16-byte aligned).
 *   variant 0  v_mfma_f32_16x16x32_bf16: 2*16*16*32 = 16384 flops each, one
 *              accumulator chain per wave (on gfx950 a dependent 16x16x32
 *              issues back to back; several independent 4-register chains
 *              make the compiler rotate accumulators with register moves
 *              that then dominate the loop);
 *   variant 1  v_mfma_f32_32x32x16_bf16: 2*32*32*16 = 32768 flops each, 8
 *              independent accumulator chains per wave.
 * Total flops = workgroups * 4 * iters * 8 * (flops per instruction).
 * Errors: GDN_ERR_NULL_POINTER, GDN_ERR_MISALIGNED, GDN_ERR_BAD_SHAPE
 * (workgroups < 1 or iters < 1), GDN_ERR_UNSUPPORTED (variant), GDN_ERR_HIP. */
gdn_status gdn_calib_mfma_loop(float* out, int32_t workgroups, int32_t iters, int32_t variant,
                               void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CALIB_H */
