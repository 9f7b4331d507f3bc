// store_util.h -- device side of the decode store (the current token's K/V
// into the pool, "SGLang 深度解读" module 5: the current K, V are written at
// their cache location before attending) and of the cascade's suffix starts,
// as jobs that any workgroups can run: the store's own launch, or the
// leading workgroups of the cascade's prefix-stage launch.
#pragma once

#include <climits>

#include "common.h"

// ---------------------------------------------------------------------------
// Suffix start of every request of a cascade call, computed once so that the
// suffix split items and the merge read one value instead of searching the
// group table themselves (a chain of dependent loads in every one of them,
// including the split items past a request's last split).  Workgroup wg of
// the n_wg that run the job takes requests wg * blockDim + t, then steps by
// n_wg * blockDim; the 64 lanes of a wave load 64 group_ptr entries at a time
// and every lane counts those <= its request (readlane broadcasts), so
// group(r) = count - 1 for ascending group_ptr; any contents give a group in
// [0, G).  Every thread of those workgroups must run it (whole waves take
// part in the search).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void suffix_starts(const SuffixStartArgs &a, unsigned wg, unsigned n_wg) {
    const int lane = threadIdx.x & 63;
    const int64_t step = (int64_t)n_wg * blockDim.x;
    for (int64_t r0 = (int64_t)wg * blockDim.x; r0 < a.batch; r0 += step) {   // uniform per workgroup
        const int64_t r = r0 + threadIdx.x;
        int cnt = 0;
        for (int base = 0; base < a.G; base += 64) {
            const int gp = base + lane < a.G ? a.group_ptr[base + lane] : INT_MAX;
            const int n = a.G - base < 64 ? a.G - base : 64;
            for (int j = 0; j < n; j++) cnt += __builtin_amdgcn_readlane(gp, j) <= r ? 1 : 0;
        }
        if (r < a.batch) {
            const int64_t P = a.group_prefix_len[cnt > 0 ? cnt - 1 : 0], L = a.seq_lens[r];
            a.lo[r] = (int32_t)(P < 0 ? 0 : (P > L ? L : P));
        }
    }
}

// The plan of a balanced suffix stage (a.plan; see SuffixStartArgs), by one
// workgroup of any whole number of waves (at most 16): thread t takes a run
// of consecutive requests, finds each one's group as suffix_starts does, and
// the runs' sums are scanned within each wave and then over the waves.
__device__ __forceinline__ int64_t plan_suffix_len(const SuffixStartArgs &a, int64_t r) {
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int base = 0; base < a.G; base += 64) {
        const int gp = base + lane < a.G ? a.group_ptr[base + lane] : INT_MAX;
        const int n = a.G - base < 64 ? a.G - base : 64;
        for (int j = 0; j < n; j++) cnt += __builtin_amdgcn_readlane(gp, j) <= r ? 1 : 0;
    }
    if (r >= a.batch) return 0;
    const int64_t L = a.seq_lens[r], row = a.req_rows[r];
    if (row < 0 || row >= a.num_rows || L <= 0) return 0;
    const int64_t P = a.group_prefix_len[cnt > 0 ? cnt - 1 : 0];
    const int64_t lo = P < 0 ? 0 : (P > L ? L : P), hi = L < a.row_stride ? L : a.row_stride;
    return hi > lo ? hi - lo : 0;
}

__device__ __forceinline__ void balanced_plan(const SuffixStartArgs &a) {
    __shared__ int64_t wave_tot[16];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, nw = blockDim.x >> 6;
    const int64_t per = ceil_div64(a.batch, blockDim.x);
    const int64_t r0 = (int64_t)t * per;
    int64_t sum = 0;
    for (int64_t i = 0; i < per; i++) sum += plan_suffix_len(a, r0 + i);   // every lane runs every step
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
    for (int64_t i = 0; i < per; i++) {
        const int64_t len = plan_suffix_len(a, r0 + i);
        if (r0 + i < a.batch) a.plan[r0 + i] = run;
        run += len;
    }
    if (t == 0) {
        int64_t total = 0;
        for (int i = 0; i < nw; i++) total += wave_tot[i];
        a.plan[a.batch] = total;
        const int64_t c = ceil_div64(total > 0 ? total : 1, a.plan_wgs);
        a.plan[a.batch + 1] = ceil_div64(c, 16) * 16;
    }
}

// ---------------------------------------------------------------------------
// FP8 codes of 16 inputs (ELT bytes each: 2 = bf16, 4 = fp32) with the factor
// sc of their KV head ("SGLang 深度拆解" section 4.3 keeps the KV cache in FP8):
// y = x / sc (fp32, IEEE division), clamped to [-448, 448], rounded to the
// nearest e4m3fn value with ties to even (v_cvt_pk_fp8_f32).
// ---------------------------------------------------------------------------
template <int ELT>
__device__ __forceinline__ uint4 quant16(const char *src, float sc) {
    float x[16];
    if (ELT == 2) {
        const uint4 a = ((const uint4 *)src)[0], b = ((const uint4 *)src)[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float4 f = ((const float4 *)src)[i];
            x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float v = x[4 * i + j] / sc;
            y[j] = v > 448.f ? 448.f : (v < -448.f ? -448.f : v);   // NaN stays NaN
        }
        int t = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        t = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], t, true);
        w[i] = (uint32_t)t;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// Decode store: token i (row i of k_new / v_new) goes to the slot at
// position lens[i] - 1 of table row req_rows[i], one 16-byte chunk of the
// pool row per thread and step (FP8: 16 codes from 16 inputs of ELT bytes);
// rows, positions and slots outside their ranges are skipped.  A thread
// loads its inputs before it looks the slot up, so the two round trips
// overlap.  Run by workgroups wg = 0 .. n_wg-1 of any size.
// ---------------------------------------------------------------------------
template <int ELT, bool FP8>
__device__ __forceinline__ void store_rows(const DecodeStoreArgs &d, unsigned wg, unsigned n_wg) {
    constexpr int NIN = FP8 ? ELT : 1;   // 16-byte input pieces per pool chunk
    const int64_t n = d.n_tokens * d.row_chunks;
    for (int64_t idx = (int64_t)wg * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)n_wg * blockDim.x) {
        const int64_t i = idx / d.row_chunks, c = idx % d.row_chunks;
        uint4 kin[NIN], vin[NIN];
#pragma unroll
        for (int j = 0; j < NIN; j++) {
            kin[j] = ((const uint4 *)d.k_new)[idx * NIN + j];
            vin[j] = ((const uint4 *)d.v_new)[idx * NIN + j];
        }
        const int64_t row = d.req_rows[i];
        const int64_t col = (int64_t)d.lens[i] - 1;
        if (row < 0 || row >= d.num_rows || col < 0 || col >= d.stride) continue;
        const int32_t s = d.r2t[row * d.stride + col];
        if (s < 0 || s >= d.num_slots) continue;
        const int64_t dst = (int64_t)s * d.row_chunks + c;
        if constexpr (FP8) {
            const int h = (int)(c / d.head_chunks);
            d.k_pool[dst] = quant16<ELT>((const char *)kin, d.k_scale[h]);
            d.v_pool[dst] = quant16<ELT>((const char *)vin, d.v_scale[h]);
        } else {
            d.k_pool[dst] = kin[0];
            d.v_pool[dst] = vin[0];
        }
    }
}

// Workgroups of the n_wg running a decode store job that compute the suffix
// starts (the rest store the tokens, so the two chains of loads run side by
// side); 0 when there are none to compute or only one workgroup, which then
// does both in turn.
__device__ __forceinline__ unsigned suffix_start_wgs(const DecodeStoreArgs &d, unsigned n_wg) {
    if (!d.ss.lo || n_wg < 2) return 0;
    const unsigned need = (unsigned)((d.ss.batch + blockDim.x - 1) / blockDim.x);
    return need < n_wg / 2 ? need : n_wg / 2;
}

// The decode store and, when d.ss.lo is set, the suffix starts, by
// workgroups wg = 0 .. n_wg-1 (whole waves).
template <int ELT, bool FP8>
__device__ __forceinline__ void decode_store_job(const DecodeStoreArgs &d, unsigned wg, unsigned n_wg) {
    const unsigned n_ss = suffix_start_wgs(d, n_wg);
    if (wg < n_ss) {
        suffix_starts(d.ss, wg, n_ss);
        return;
    }
    store_rows<ELT, FP8>(d, wg - n_ss, n_wg - n_ss);
    if (d.ss.lo && n_ss == 0) suffix_starts(d.ss, wg, n_wg);
}
