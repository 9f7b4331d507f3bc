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

// ---- balanced suffix stage ----------------------------------------------------
// The suffix items above are (request, split) pairs: their lengths follow
// the suffixes, and as the grid drains fewer and fewer compute units keep
// gathers in flight.  Here the suffixes of all requests are laid end to end
// and every workgroup of a head group takes an equal run of that sequence
// (plan: the runs' starts, from sk_plan_kernel), whatever requests it
// crosses: each piece -- a run's part inside one request -- leaves a partial
// state of its own (row request + run, see sk_state_rows), which the merge
// finds from the same plan.

// Suffix length of request r (0 for a row outside the table), as rows_split
// bounds it: keys [suffix_lo[r], min(seq_lens[r], row_stride)).
__device__ __forceinline__ int64_t sk_suffix_len(const SplitArgs &a, int r) {
    const int64_t L = a.seq_lens[r], row = a.req_rows[r];
    if (row < 0 || row >= a.num_rows || L <= 0) return 0;
    const int64_t P = a.suffix_lo[r];
    const int64_t lo = P < 0 ? 0 : (P > L ? L : P), hi = L < a.row_stride ? L : a.row_stride;
    return hi > lo ? hi - lo : 0;
}

// plan[r] = sum of the suffix lengths of requests before r (r <= batch),
// plan[batch + 1] = keys per workgroup: the total over sk_wgs, rounded up to
// a whole tile.  One workgroup of 1024 threads; thread t sums a run of
// consecutive requests, the runs are scanned within each wave and then over
// the waves.
__global__ void __launch_bounds__(1024) sk_plan_kernel(SplitArgs a, int64_t *plan) {
    __shared__ int64_t wave_tot[16];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int per = (a.batch + 1023) / 1024;
    const int r0 = min(t * per, a.batch), r1 = min(r0 + per, a.batch);
    int64_t sum = 0;
    for (int r = r0; r < r1; r++) sum += sk_suffix_len(a, r);
    int64_t x = sum;                                 // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int64_t run = x - sum;
    for (int i = 0; i < wv; i++) run += wave_tot[i];
    for (int r = r0; r < r1; r++) {
        plan[r] = run;
        run += sk_suffix_len(a, r);
    }
    if (t == 1023) {
        int64_t total = 0;
        for (int i = 0; i < 16; i++) total += wave_tot[i];
        plan[a.batch] = total;
        const int64_t c = ceil_div64(total > 0 ? total : 1, a.sk_wgs);
        plan[a.batch + 1] = ceil_div64(c, 16) * 16;
    }
}

// Workgroup id = w * (Hkv / HPW) + head group: run w of the concatenated
// suffixes for the head group's KV heads.
// Four workgroups per compute unit (all of the grid at once): at most 128
// VGPRs, and, as in split_rows_loop_kernel, each piece takes the thread id
// and the arguments through values the compiler cannot see through, so that
// nothing derived from them stays live across the loop.
template <int D, bool FP8, int HPW>
__global__ void __launch_bounds__(64 * HPW, 4) split_rows_balanced_kernel(SplitArgs a) {
    constexpr int TB = (FP8 ? 32 : 16) * HPW * D * (FP8 ? 1 : 2);   // bytes of one K (or V) tile
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[TB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[TB];
    extern __shared__ int32_t slot_lds[];  // [chunk]
    const int ng = a.Hkv / HPW;
    const int hg = (int)(blockIdx.x % (unsigned)ng);
    const int64_t w = blockIdx.x / (unsigned)ng;
    const int64_t *plan = a.sk_plan;
    const int64_t total = plan[a.batch], C = plan[a.batch + 1];
    int64_t p = w * C;
    const int64_t end = p + C < total ? p + C : total;
    if (p >= end) return;
    // the request holding key p: the last r < batch with plan[r] <= p (plan
    // ascends from plan[0] = 0); 64 entries per ballot
    const int lane = threadIdx.x & 63;
    int r = -1;
    for (int base = 0; base < a.batch; base += 64) {
        const int i = base + lane;
        const int c = __popcll(__builtin_amdgcn_ballot_w64(i < a.batch && plan[i] <= p));
        r += c;
        if (c < 64) break;
    }
    for (;;) {
        const int64_t r_off = plan[r], r_end = plan[r + 1];
        const int64_t pe = end < r_end ? end : r_end;
        const int64_t L = a.seq_lens[r], P = a.suffix_lo[r];
        const int64_t lo = P < 0 ? 0 : (P > L ? L : P);
        int tid = (int)threadIdx.x;
        typedef const __attribute__((address_space(4))) SplitArgs *KArgs;
        KArgs ap = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+v"(tid), "+s"(ap));
        rows_segment<D, FP8, HPW, true>(*(const SplitArgs *)ap, tid, r, hg, a.req_rows[r], lo + (p - r_off),
                                        (int)(pe - p), r + w, k_lds, v_lds, slot_lds);
        p = pe;
        if (p >= end) break;
        while (plan[r + 1] <= p) r++;              // the next request with keys (plan[batch] > p)
        __syncthreads();                            // tiles and slot table free for the next piece
    }
}

}  // namespace

// Balanced suffix stage (kind 2 with suffix_lo): sk_plan_kernel writes plan
// (batch + 2 int64), then a.sk_wgs workgroups per head group of kRowsHeads KV
// heads take equal runs of the concatenated suffixes, writing states to rows
// request + run of a.part (sk_state_rows(batch, sk_wgs) rows, S = 1).
int launch_split_rows_balanced(const SplitArgs &a0, bool fp8, int64_t *plan, hipStream_t st) {
    if (a0.kind != 2 || !a0.suffix_lo || !plan || a0.sk_wgs < 1 || a0.part.S != 1) return SGL_ERR_INVALID;
    if (a0.Hkv % kRowsHeads != 0 || a0.Hkv > 16 || a0.Hq / a0.Hkv > 16) return SGL_ERR_UNSUPPORTED;
    if (a0.batch == 0) return SGL_OK;
    if (a0.chunk % (fp8 ? 32 : 16) != 0) return SGL_ERR_INVALID;
    if (fp8 && (!a0.k_scale || !a0.v_scale)) return SGL_ERR_INVALID;
    SplitArgs a = a0;
    a.sk_plan = plan;
    hipLaunchKernelGGL(sk_plan_kernel, dim3(1), dim3(1024), 0, st, a, plan);
    const int64_t n_wg = (int64_t)a.sk_wgs * (a.Hkv / kRowsHeads);
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
    const dim3 grid((unsigned)n_wg), block(64 * kRowsHeads);
    if (a.D == 128) {
        if (fp8) hipLaunchKernelGGL((split_rows_balanced_kernel<128, true, kRowsHeads>), grid, block, dyn, st, a);
        else hipLaunchKernelGGL((split_rows_balanced_kernel<128, false, kRowsHeads>), grid, block, dyn, st, a);
    } else {
        if (fp8) hipLaunchKernelGGL((split_rows_balanced_kernel<64, true, kRowsHeads>), grid, block, dyn, st, a);
        else hipLaunchKernelGGL((split_rows_balanced_kernel<64, false, kRowsHeads>), grid, block, dyn, st, a);
    }
    return hip_status(hipGetLastError());
}

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
