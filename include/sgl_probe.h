/*
 * sgl_probe.h -- measurement helpers of libsgl_attn.so: what the chip in
 * hand actually sustains, so that a kernel's roofline fraction can be read
 * against the measured ceiling as well as against the published peak
 * (MI355X: 8 TB/s of HBM3E, 2.5 PFLOP/s of dense bf16 MFMA).  Neither call is
 * part of the attention method; they compute nothing a caller needs.
 *
 * Conventions as in sgl_attn.h: plain C types, device pointers to GPU memory
 * that the caller owns, streams as void* (NULL = the default stream), work
 * only enqueued, an sgl_status returned, argument checks before any GPU work.
 */
#ifndef SGL_PROBE_H
#define SGL_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core rate.  n_wg workgroups of 4 waves; every wave runs
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 accumulations
 * (A = B = x rounded to bf16, every element), so a launch performs exactly
 * n_wg * 4 * iters * 8 * 32768 floating-point operations.  out (device,
 * float32, n_wg * 256 entries, caller-owned) receives, per lane, the sum of
 * element 0 of its 8 accumulators: 8 * 16 * iters * bf16(x)^2, exact in fp32
 * while that stays below 2^24 (so a caller can check the work was done).
 * Errors: SGL_ERR_INVALID for n_wg < 1, iters < 1 or out == NULL;
 * SGL_ERR_HIP if the launch fails. */
int sgl_probe_mfma_bf16(int32_t n_wg, int32_t iters, float x, float *out, void *stream);

/* Streaming copy bandwidth: dst[i] = src[i] for `bytes` bytes (device
 * buffers, 16-byte aligned, not overlapping), each byte read once and
 * written once.  Errors: SGL_ERR_INVALID for bytes < 0, bytes not a multiple
 * of 16, a misaligned or NULL pointer with bytes > 0, or overlapping
 * buffers; SGL_ERR_UNSUPPORTED beyond 32 TiB (2^31 workgroups of 16 KiB);
 * SGL_ERR_HIP if the launch fails.  bytes == 0 enqueues nothing. */
int sgl_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SGL_PROBE_H */
