// kernels_probe.hip -- the two measurement helpers of sgl_probe.h: the
// dense bf16 MFMA rate and the streaming copy bandwidth of the chip in hand,
// the ceilings the attention kernels' roofline fractions are read against
// next to the published MI355X peaks.
#include "common.h"
#include "sgl_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 8;      // independent accumulators per wave
constexpr int kCopyUnroll = 4;       // 16-byte loads in flight per thread before its stores

// Each wave: iters rounds of kProbeChains independent 32x32x16 bf16 MFMAs, so
// consecutive MFMAs never wait on one another and the matrix pipe of every
// SIMD stays busy (the workgroup's four waves spread over the CU's four
// SIMDs).  The operands come from a kernel argument, so nothing folds.
__global__ void __launch_bounds__(kProbeThreads) mfma_probe_kernel(int iters, float x, float *out) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = (__bf16)x;
    f32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; c++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[c][e] = 0.f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int c = 0; c < kProbeChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; c++) s += acc[c][0];
    out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// dst = src over n 16-byte chunks: workgroup b copies the contiguous chunks
// [b * 256 * kCopyUnroll, (b + 1) * 256 * kCopyUnroll), each thread issuing
// its kCopyUnroll non-temporal loads before its stores (the fastest of the
// block, grid-stride, unroll and cache-hint variants measured on MI355X).
__global__ void __launch_bounds__(kProbeThreads) copy_probe_kernel(const u32x4 *__restrict__ src,
                                                                   u32x4 *__restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kProbeThreads * kCopyUnroll + threadIdx.x;
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + u * kProbeThreads;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + u * kProbeThreads;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

}  // namespace

extern "C" int sgl_probe_mfma_bf16(int32_t n_wg, int32_t iters, float x, float *out, void *stream) {
    if (n_wg < 1 || iters < 1 || !out) return SGL_ERR_INVALID;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)n_wg), dim3(kProbeThreads), 0, (hipStream_t)stream, iters,
                       x, out);
    return hip_status(hipGetLastError());
}

extern "C" int sgl_probe_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    if (bytes < 0 || bytes % 16 != 0) return SGL_ERR_INVALID;
    if (bytes == 0) return SGL_OK;
    if (!src || !dst || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return SGL_ERR_INVALID;
    const int64_t n = bytes / 16;
    const char *s = (const char *)src, *d = (const char *)dst;
    if (s < d + bytes && d < s + bytes) return SGL_ERR_INVALID;   // overlapping
    const int64_t per_wg = (int64_t)kProbeThreads * kCopyUnroll;
    const int64_t wg = (n + per_wg - 1) / per_wg;
    if (wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)wg), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)src, (u32x4 *)dst, n);
    return hip_status(hipGetLastError());
}
