/*
 * mla_probe.h -- C ABI of the measurement probes shipped beside the MLA library
 * (libmla_probe.so).  They are not part of the decode path: bench.py uses them to
 * measure the achievable HBM read bandwidth and bf16 MFMA rate of the GPU it runs
 * on, so that the decode kernels' rates can be reported against measured as well as
 * published peaks.
 *
 * Both calls enqueue one kernel on `stream` (a hipStream_t, NULL = default) and
 * return without synchronising; the caller times them with events.  All pointers
 * are device pointers owned by the caller.  Statuses are those of mla.h.
 */
#ifndef MLA_PAGED_LATENT_MLA_PROBE_H
#define MLA_PAGED_LATENT_MLA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_probe_hbm_read -- read `bytes` bytes of `src` once, 16 bytes per lane per load
 * with several loads in flight per lane, over a grid of 8 workgroups of 256 threads per
 * compute unit; each thread folds what it read into one 16-byte value written to
 * `sink` (so the loads cannot be dropped).
 *
 *   src    device buffer, 16-byte aligned, bytes a multiple of 16
 *   sink   device buffer of at least mla_probe_sink_bytes() bytes, 16-byte aligned
 *
 * Achievable read bandwidth = bytes / kernel time.  MLA_ERR_ALIGN for misaligned
 * pointers or sizes, MLA_ERR_NULL for NULL, MLA_ERR_HIP on launch failure.
 */
mla_status_t mla_probe_hbm_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * mla_probe_mfma_bf16 -- `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * chains per wave, 8 waves (two per SIMD) per compute unit, register operands only;
 * each thread writes one float of its accumulators to `sink`.
 *
 *   flops = compute units * 8 waves * iters * 4 * 32 * 32 * 16 * 2
 *   (mla_probe_mfma_flops() returns it for the current device)
 *
 * 1 <= iters <= 2^24.  MLA_ERR_SHAPE outside that range.
 */
mla_status_t mla_probe_mfma_bf16(float* sink, int32_t iters, void* stream);

/* bytes `sink` must hold for either probe on the current device (0 on error) */
size_t mla_probe_sink_bytes(void);

/* floating-point operations of one mla_probe_mfma_bf16 call on the current device */
double mla_probe_mfma_flops(int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_LATENT_MLA_PROBE_H */
