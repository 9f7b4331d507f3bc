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
    rows_split<D, FP8, HPW>(a, (int)blockIdx.x, (int)threadIdx.x, k_lds, v_lds, slot_lds);
}

// The suffix stage over a grid of a.rounds split rounds (sized for the
// expected suffixes).  A workgroup first runs its own item, then the items
// bid + k * gridDim.x, k >= 1, that have keys -- rounds s + k * a.rounds of a
// grid of all max_splits rounds, on the same XCD (gridDim.x is a multiple of
// 8).  The lanes test 64 such items at a time; every wave finds the same
// ones.  One call site of rows_split, and each pass takes the thread id and
// the arguments through values the compiler cannot see through, so nothing
// derived from them stays live across the loop.
template <int D, bool FP8, int HPW>
__global__ void __launch_bounds__(64 * HPW) split_rows_loop_kernel(SplitArgs a) {
    constexpr int TB = (FP8 ? 32 : 16) * HPW * D * (FP8 ? 1 : 2);   // bytes of one K (or V) tile
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[TB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[TB];
    extern __shared__ int32_t slot_lds[];  // [chunk]
    const int bid = (int)blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int64_t step = gridDim.x;
    int item = bid;
    int64_t k0 = 1;          // first later item not yet tested
    uint64_t mask = 0;       // tested items k0 - 64 + l with keys, not yet run
    for (;;) {
        int tid = (int)threadIdx.x;
        typedef const __attribute__((address_space(4))) SplitArgs *KArgs;
        KArgs ap = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+v"(tid), "+s"(ap));
        rows_split<D, FP8, HPW>(*(const SplitArgs *)ap, item, tid, k_lds, v_lds, slot_lds);
        while (!mask) {
            if (bid + k0 * step > 0x7fffffff) return;
            int s0, v0;
            rows_item(a, HPW, (int)(bid + k0 * step), s0, v0);
            if (s0 >= a.max_splits) return;
            const int64_t vid = bid + (k0 + lane) * step;
            mask = __builtin_amdgcn_ballot_w64(vid <= 0x7fffffff && rows_item_live(a, HPW, (int)vid));
            k0 += 64;
        }
        const int l = __builtin_ctzll(mask);
        mask &= mask - 1;
        item = (int)(bid + (k0 - 64 + l) * step);
        __syncthreads();     // the previous item is done with the tiles and the slot table
    }
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
    if (a.rounds > 0 && (a.kind != 2 || !a.suffix_lo)) return SGL_ERR_INVALID;
    const int64_t rounds = a.rounds > 0 && a.rounds < a.max_splits ? a.rounds : a.max_splits;
    const int64_t per_round = 8 * (((n_v + rb - 1) / rb + 7) / 8) * rb;
    if (per_round * a.max_splits > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const int64_t n_wg = per_round * rounds;
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
    const dim3 grid((unsigned)n_wg), block(64 * hpw);
    SplitArgs x = a;
    x.rounds = rounds < a.max_splits ? (int32_t)rounds : 0;
#define SGL_ROWS(DD, F8, H)                                                                                  \
    do {                                                                                                     \
        if (x.rounds > 0) hipLaunchKernelGGL((split_rows_loop_kernel<DD, F8, H>), grid, block, dyn, st, x); \
        else hipLaunchKernelGGL((split_rows_kernel<DD, F8, H>), grid, block, dyn, st, x);                  \
    } while (0)
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
