// kernels_f32.hip -- fp32 attention (extend, and split partial states for
// decode / cascade).  One wave per (query row, q head) walks its keys in
// blocks of 64 with the online softmax ("SGLang 深度拆解" (chenxutan.com)
// section 3.2, PagedPrefill: running maximum, rescaled sum and accumulator),
// one block at a time instead of one key at a time, so that a block costs a
// few memory round trips rather than one per key: lane j owns key j of the
// block for the scores (its whole K row, against the query broadcast from
// LDS), then for P V lane d owns head dims d (and d + 64) and adds the 64
// keys' V rows, whose loads all go out before the sums.  Full fp32
// arithmetic throughout; this path serves small fp32 workloads, the bf16
// path is the tuned one.
#include "common.h"

template <int PER>
struct RangeState {
    float m, l;
    float acc[PER];
};

// Attend one query vector (lane holds elements lane*PER .. lane*PER+PER-1) to
// keys [lo, hi) of a req_to_token row.  m is in log2 units of the scaled
// score.  Every lane of the wave must be active.
template <int PER>
__device__ RangeState<PER> attend_range_f32(const float *qv, const float *__restrict__ k_pool,
                                            const float *__restrict__ v_pool, int64_t num_slots,
                                            const int32_t *__restrict__ row, int64_t lo, int64_t hi,
                                            int kvh, int Hkv, float qscale) {
    constexpr int D = PER * 64;
    const int lane = threadIdx.x & 63;
    __shared__ float q_lds[D];
#pragma unroll
    for (int i = 0; i < PER; i++) q_lds[lane * PER + i] = qv[i];
    __syncthreads();
    RangeState<PER> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int i = 0; i < PER; i++) st.acc[i] = 0.f;
    constexpr int VC = 32;                                            // V rows in flight per lane
    for (int64_t j0 = lo; j0 < hi; j0 += 64) {
        const int nv = (int)(hi - j0 < 64 ? hi - j0 : 64);           // keys in this block (uniform)
        const bool valid = lane < nv;
        const int32_t slot = valid ? safe_slot(row[j0 + lane], num_slots) : 0;
        // this lane's key: s = q . k over the whole row
        const float4 *kr = (const float4 *)(k_pool + ((int64_t)slot * Hkv + kvh) * D);
        float sc = 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; c++) {
            const float4 k4 = kr[c];
            const float4 q4 = *(const float4 *)(q_lds + 4 * c);
            sc = fmaf(q4.x, k4.x, sc);
            sc = fmaf(q4.y, k4.y, sc);
            sc = fmaf(q4.z, k4.z, sc);
            sc = fmaf(q4.w, k4.w, sc);
        }
        sc = valid ? sc * qscale : -INFINITY;
        const float m_new = fmaxf(st.m, wave_max(sc));               // finite: the block has a key
        const float alpha = exp2f(st.m - m_new);
        const float p = valid ? exp2f(sc - m_new) : 0.f;
        st.l = st.l * alpha + wave_sum(p);
#pragma unroll
        for (int i = 0; i < PER; i++) st.acc[i] *= alpha;
        // P V: VC keys at a time, their V rows loaded before any is added
        for (int c0 = 0; c0 < nv; c0 += VC) {
            float vv[VC][PER];
#pragma unroll
            for (int u = 0; u < VC; u++) {
                if (c0 + u < nv) {
                    const int64_t sj = __builtin_amdgcn_readlane(slot, c0 + u);
                    const float *vr = v_pool + (sj * Hkv + kvh) * D + lane * PER;
#pragma unroll
                    for (int i = 0; i < PER; i++) vv[u][i] = vr[i];
                }
            }
#pragma unroll
            for (int u = 0; u < VC; u++) {
                if (c0 + u < nv) {
                    const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), c0 + u));
#pragma unroll
                    for (int i = 0; i < PER; i++) st.acc[i] = fmaf(pj, vv[u][i], st.acc[i]);
                }
            }
        }
        st.m = m_new;
    }
    return st;
}

template <int PER>
__global__ void __launch_bounds__(64) extend_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k_pool, const float *__restrict__ v_pool,
    int64_t num_slots, const int32_t *__restrict__ r2t, int64_t num_rows, int64_t stride,
    const int32_t *__restrict__ req_rows, const int32_t *__restrict__ prefix_lens,
    const int64_t *__restrict__ q_off, int Hq, int Hkv, float qscale, float *__restrict__ o,
    float *__restrict__ lse) {
    constexpr int D = PER * 64;
    const int i = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
    const int lane = threadIdx.x;
    const int64_t t0 = q_off[r], E = q_off[r + 1] - t0;
    if (i >= E) return;
    const int64_t rowi = req_rows[r];
    const int64_t P = prefix_lens[r];
    if (rowi < 0 || rowi >= num_rows || P < 0) return;
    const int64_t pos = P + i;                 // absolute position of this query
    const int64_t hi = pos + 1 < stride ? pos + 1 : stride;   // keys j <= pos
    const int kvh = h / (Hq / Hkv);
    const int64_t tok = t0 + i;
    float qv[PER];
#pragma unroll
    for (int e = 0; e < PER; e++) qv[e] = q[(tok * Hq + h) * D + lane * PER + e];
    RangeState<PER> st = attend_range_f32<PER>(qv, k_pool, v_pool, num_slots, r2t + rowi * stride,
                                               0, hi, kvh, Hkv, qscale);
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
#pragma unroll
    for (int e = 0; e < PER; e++) o[(tok * Hq + h) * D + lane * PER + e] = st.acc[e] * inv;
    if (lse && lane == 0) lse[tok * Hq + h] = st.l > 0.f ? (st.m + log2f(st.l)) * kLn2 : -INFINITY;
}

int launch_extend_f32(const float *q, const float *k_pool, const float *v_pool, int64_t num_slots,
                      const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                      const int32_t *req_rows, const int32_t *prefix_lens, const int64_t *q_off,
                      int32_t batch, int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D,
                      float scale, float *o, float *lse, hipStream_t st) {
    if (batch == 0 || max_extend_len == 0) return SGL_OK;
    dim3 grid(max_extend_len, Hq, batch), block(64);
    const float qs = scale * kLog2e;
    if (D == 128)
        hipLaunchKernelGGL(extend_f32_kernel<2>, grid, block, 0, st, q, k_pool, v_pool, num_slots,
                           r2t, num_rows, row_stride, req_rows, prefix_lens, q_off, Hq, Hkv, qs, o, lse);
    else
        hipLaunchKernelGGL(extend_f32_kernel<1>, grid, block, 0, st, q, k_pool, v_pool, num_slots,
                           r2t, num_rows, row_stride, req_rows, prefix_lens, q_off, Hq, Hkv, qs, o, lse);
    return hip_status(hipGetLastError());
}

__device__ __forceinline__ int find_group_f32(const int32_t *group_ptr, int G, int r) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (group_ptr[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Partial state of one (request, q head, split).  Grid (max_splits, Hq, batch).
template <int PER>
__global__ void __launch_bounds__(64) split_f32_kernel(SplitArgs a) {
    constexpr int D = PER * 64;
    const int s = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
    const int lane = threadIdx.x;
    const int64_t L = a.seq_lens[r];
    int64_t lo, hi;
    int64_t ref_row;
    if (a.kind == 0) {
        lo = 0; hi = L; ref_row = a.req_rows[r];
    } else {
        const int g = find_group_f32(a.group_ptr, a.G, r);
        int64_t P = a.group_prefix_len[g];
        P = P < 0 ? 0 : (P > L ? L : P);
        if (a.kind == 1) { lo = 0; hi = P; ref_row = a.req_rows[a.group_ptr[g]]; }
        else { lo = P; hi = L; ref_row = a.req_rows[r]; }
    }
    const int64_t n_split = ceil_div64(hi - lo, a.chunk);
    if (s >= n_split || s >= a.part.S) return;
    if (ref_row < 0 || ref_row >= a.num_rows) return;
    const int64_t k0 = lo + (int64_t)s * a.chunk;
    int64_t k1 = k0 + a.chunk < hi ? k0 + a.chunk : hi;
    if (k1 > a.row_stride) k1 = a.row_stride;
    const int kvh = h / (a.Hq / a.Hkv);
    const float *q = (const float *)a.q;
    float qv[PER];
#pragma unroll
    for (int e = 0; e < PER; e++) qv[e] = q[((int64_t)r * a.Hq + h) * D + lane * PER + e];
    RangeState<PER> st = attend_range_f32<PER>(qv, (const float *)a.k_pool, (const float *)a.v_pool,
                                               a.num_slots, a.r2t + ref_row * a.row_stride, k0, k1,
                                               kvh, a.Hkv, a.scale * kLog2e);
    const int64_t idx = ((int64_t)r * a.part.S + s) * a.Hq + h;
#pragma unroll
    for (int e = 0; e < PER; e++) a.part.o[idx * D + lane * PER + e] = st.acc[e];
    if (lane == 0) {
        a.part.ml[idx * 2] = st.m;
        a.part.ml[idx * 2 + 1] = st.l;
    }
}

int launch_split_f32(const SplitArgs &a, hipStream_t st) {
    if (a.batch == 0 || a.max_splits == 0) return SGL_OK;
    dim3 grid(a.max_splits, a.Hq, a.batch), block(64);
    if (a.D == 128) hipLaunchKernelGGL(split_f32_kernel<2>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(split_f32_kernel<1>, grid, block, 0, st, a);
    return hip_status(hipGetLastError());
}
