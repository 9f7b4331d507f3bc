// kernels_decode_rows.hip -- split-K decode for the flat call and the cascade
// suffix, one workgroup per (request, key split, group of up to 4 KV heads)
// loading whole rows of the group's heads (the work item is rows_split in
// decode_rows.h).
#include "common.h"
#include "decode_rows.h"

namespace {

using namespace sgl_decode;

template <int D, bool FP8, int HPW>
__global__ void __launch_bounds__(64 * HPW) split_rows_kernel(SplitArgs a) {
    constexpr int TB = (FP8 ? 32 : 16) * HPW * D * (FP8 ? 1 : 2);   // bytes of one K (or V) tile
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[TB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[TB];
    extern __shared__ int32_t slot_lds[];  // [chunk]
    rows_split<D, FP8, HPW>(a, (int)blockIdx.x, k_lds, v_lds, slot_lds);
}

}  // namespace

// Flat (kind 0) or suffix (kind 2) splits with whole-row loads of head
// groups of kRowsHeads KV heads (all of them when Hkv is smaller).  Returns
// SGL_ERR_UNSUPPORTED for shapes it does not cover (Hkv not 2, 4, 8 or 16),
// which the per-head kernels handle.
int launch_split_rows(const SplitArgs &a, bool fp8, hipStream_t st) {
    if (a.kind != 0 && a.kind != 2) return SGL_ERR_UNSUPPORTED;
    if (a.Hkv != 2 && a.Hkv != 4 && a.Hkv != 8 && a.Hkv != 16) return SGL_ERR_UNSUPPORTED;
    if (a.Hq / a.Hkv > 16) return SGL_ERR_UNSUPPORTED;
    if (a.n_sets == 0 || a.max_splits == 0) return SGL_OK;
    if (a.chunk % (fp8 ? 32 : 16) != 0 || a.xcd_block < 1) return SGL_ERR_INVALID;
    if (fp8 && (!a.k_scale || !a.v_scale)) return SGL_ERR_INVALID;
    const int hpw = a.Hkv < kRowsHeads ? a.Hkv : kRowsHeads;
    const int rb = a.xcd_block;
    const int64_t n_v = (int64_t)a.n_sets * (a.Hkv / hpw);
    const int64_t n_wg = 8 * (((n_v + rb - 1) / rb + 7) / 8) * rb * a.max_splits;
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
    const dim3 grid((unsigned)n_wg), block(64 * hpw);
#define SGL_ROWS(DD, F8, H) hipLaunchKernelGGL((split_rows_kernel<DD, F8, H>), grid, block, dyn, st, a)
#define SGL_ROWS_H(DD, F8) \
    do { if (hpw == 8) SGL_ROWS(DD, F8, 8); else if (hpw == 4) SGL_ROWS(DD, F8, 4); else SGL_ROWS(DD, F8, 2); } while (0)
    if (a.D == 128) {
        if (fp8) SGL_ROWS_H(128, true); else SGL_ROWS_H(128, false);
    } else {
        if (fp8) SGL_ROWS_H(64, true); else SGL_ROWS_H(64, false);
    }
#undef SGL_ROWS_H
#undef SGL_ROWS
    return hip_status(hipGetLastError());
}
