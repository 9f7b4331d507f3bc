// kernels_decode.hip -- bf16 split-K decode attention for gfx950.
//
// One wave per (KV head, split, request-or-group).  The wave owns up to
// 16*NB query rows that read the same KV head: the g = Hq/Hkv query heads of
// one request (flat decode, cascade suffix), or the g heads of every request
// of a group (cascade prefix: the shared prefix is read once for all of the
// group's queries).  For each 32-key tile of its split it
//   1. gathers the K rows of the tile straight into MFMA operand registers
//      (lane = key x quarter of head_dim, 64 contiguous bytes per lane);
//   2. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on M, query
//      rows on N);
//   3. updates the running max / sum per row (online softmax, the update of
//      "SGLang 深度拆解" (chenxutan.com) section 3.2 applied to a tile);
//   4. gathers the V rows into LDS row-major and reads them back transposed
//      with ds_read_b64_tr_b16, so O^T += V^T P^T runs on MFMA as well, with
//      P^T taken directly from the S^T accumulator registers (the key order
//      inside each MFMA is chosen so that no lane exchange is needed).
// The split's state (m, l, unnormalised o) goes to the workspace; a merge
// kernel combines the splits of a request (and, for the cascade, its group's
// prefix splits) with the log-sum-exp rule.
#include "common.h"

namespace {

constexpr int TILE = 32;   // keys per tile

template <int D>
struct DecodeLds {
    static constexpr int kRowBytes = D * 2 + 32;               // padded V row (bank spread)
    static constexpr int kVBytes = TILE * kRowBytes;
};

__device__ __forceinline__ int find_group_dec(const int32_t *group_ptr, int G, int r) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (group_ptr[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
    union { uint4 u; bf16x8 b; } x;
    x.u = u;
    return x.b;
}

template <int D, int NB>
__global__ void __launch_bounds__(64) split_bf16_kernel(SplitArgs a) {
    constexpr int QT = D / 32;          // MFMA k-steps over head_dim
    constexpr int DB = D / 16;          // 16-dim output blocks
    constexpr int ROWB = DecodeLds<D>::kRowBytes;
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[DecodeLds<D>::kVBytes];
    extern __shared__ int32_t slot_lds[];  // [chunk]

    const int lane = threadIdx.x;
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int n_rb = a.kind == 1 ? a.row_blocks : 1;   // 16*NB-row blocks of a big group
    const int set = blockIdx.z / n_rb;
    const int rb = blockIdx.z % n_rb;
    const int g = a.Hq / a.Hkv;

    // ---- which rows, which keys ----------------------------------------------
    int first_req, n_members;
    int64_t lo, hi, ref_row;
    if (a.kind == 1) {
        const int grp = set;
        first_req = a.group_ptr[grp];
        n_members = a.group_ptr[grp + 1] - first_req;
        if (n_members <= 0 || first_req < 0 || first_req + n_members > a.batch) return;
        int64_t P = a.group_prefix_len[grp];
        lo = 0;
        hi = P < 0 ? 0 : P;
        ref_row = a.req_rows[first_req];
    } else {
        first_req = set;
        n_members = 1;
        const int64_t L = a.seq_lens[set];
        ref_row = a.req_rows[set];
        if (a.kind == 0) {
            lo = 0;
        } else {
            const int grp = find_group_dec(a.group_ptr, a.G, set);
            int64_t P = a.group_prefix_len[grp];
            lo = P < 0 ? 0 : (P > L ? L : P);
        }
        hi = L;
    }
    const int row_base = rb * 16 * NB;              // first group row of this wave
    const int rows = n_members * g - row_base;      // rows left from row_base on
    if (rows <= 0) return;
    if (ref_row < 0 || ref_row >= a.num_rows) return;
    if (hi > a.row_stride) hi = a.row_stride;
    const int64_t n_split = ceil_div64(hi - lo, a.chunk);
    if (s >= n_split || s >= a.part.S) return;
    const int64_t k0 = lo + (int64_t)s * a.chunk;
    const int64_t k1 = k0 + a.chunk < hi ? k0 + a.chunk : hi;
    const int nk = (int)(k1 - k0);

    const int32_t *row = a.r2t + ref_row * a.row_stride;
    for (int j = lane; j < nk; j += 64) slot_lds[j] = safe_slot(row[k0 + j], a.num_slots);

    const __bf16 *q = (const __bf16 *)a.q;
    const __bf16 *kp = (const __bf16 *)a.k_pool;
    const __bf16 *vp = (const __bf16 *)a.v_pool;
    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand: lane (row n16, quarter kq) holds dims (D/4)kq + 8t + i --
    bf16x8 qf[NB][QT];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int rho = nb * 16 + n16;
        if (rho < rows) {
            const int req = first_req + (row_base + rho) / g;
            const int h = kvh * g + (row_base + rho) % g;
            const uint4 *src = (const uint4 *)(q + ((int64_t)req * a.Hq + h) * D + (D / 4) * kq);
#pragma unroll
            for (int t = 0; t < QT; t++) qf[nb][t] = as_bf16x8(src[t]);
        } else {
#pragma unroll
            for (int t = 0; t < QT; t++) qf[nb][t] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }

    f32x4 oacc[DB][NB];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) oacc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) { m_run[nb] = -INFINITY; l_run[nb] = 0.f; }

    const float qscale = a.scale * kLog2e;
    const int64_t rowstride_el = (int64_t)a.Hkv * D;
    __syncthreads();

    for (int t0 = 0; t0 < nk; t0 += TILE) {
        // ---- gather K (registers) and V (registers, then LDS) ---------------
        uint4 kf[2][QT];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int kk = t0 + kb * 16 + n16;
            if (kk < nk) {
                const uint4 *src = (const uint4 *)(kp + (int64_t)slot_lds[kk] * rowstride_el +
                                                   kvh * D + (D / 4) * kq);
#pragma unroll
                for (int t = 0; t < QT; t++) kf[kb][t] = src[t];
            } else {
#pragma unroll
                for (int t = 0; t < QT; t++) kf[kb][t] = make_uint4(0, 0, 0, 0);
            }
        }
        constexpr int VCH = D / 16;    // uint4 per lane: half a row (lane = key*2 + half)
        uint4 vf[VCH];
        {
            const int kk = t0 + (lane >> 1);
            if (kk < nk) {
                const uint4 *src = (const uint4 *)(vp + (int64_t)slot_lds[kk] * rowstride_el +
                                                   kvh * D + (lane & 1) * (D / 2));
#pragma unroll
                for (int c = 0; c < VCH; c++) vf[c] = src[c];
            } else {
#pragma unroll
                for (int c = 0; c < VCH; c++) vf[c] = make_uint4(0, 0, 0, 0);
            }
        }

        // ---- S^T = K Q^T ------------------------------------------------------
        f32x4 sacc[2][NB];
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < QT; t++)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kb][t]), qf[nb][t], c, 0, 0, 0);
                sacc[kb][nb] = c;
            }

        // ---- V tile -> LDS (row-major, padded rows) ------------------------------
        {
            unsigned char *dst = v_lds + (lane >> 1) * ROWB + (lane & 1) * D;
#pragma unroll
            for (int c = 0; c < VCH; c++) *(uint4 *)(dst + c * 16) = vf[c];
        }

        // ---- online softmax per row ------------------------------------------------
        bf16x8 pf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            float sv[2][4];
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int kk = t0 + kb * 16 + kq * 4 + j;
                    float x = sacc[kb][nb][j] * qscale;
                    x = kk < nk ? x : -INFINITY;
                    sv[kb][j] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[nb], mx);
            const float alpha = exp2f(m_run[nb] - m_new);   // 0 when m_run = -inf
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float p = exp2f(sv[kb][j] - m_new);
                    psum += p;
                    pf[nb][kb * 4 + j] = (__bf16)p;
                }
            l_run[nb] = l_run[nb] * alpha + psum;
            m_run[nb] = m_new;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db][nb] *= alpha;
        }

        __syncthreads();   // V tile visible

        // ---- O^T += V^T P^T ---------------------------------------------------
        const int r4 = n16 >> 2, qq = n16 & 3;
#pragma unroll
        for (int db = 0; db < DB; db++) {
            const SGL_LDS i16x4 *p0 =
                (const SGL_LDS i16x4 *)(v_lds + (kq * 4 + r4) * ROWB + (db * 16 + qq * 4) * 2);
            const SGL_LDS i16x4 *p1 =
                (const SGL_LDS i16x4 *)(v_lds + (16 + kq * 4 + r4) * ROWB + (db * 16 + qq * 4) * 2);
            i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p0);
            i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p1);
            union { i16x4 h[2]; bf16x8 b; } va;
            va.h[0] = lo4;
            va.h[1] = hi4;
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
                oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.b, pf[nb], oacc[db][nb], 0, 0, 0);
        }
        __syncthreads();   // V tile consumed before the next overwrite
    }

    // ---- write the split's state ---------------------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        float l = l_run[nb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int rho = nb * 16 + n16;
        if (rho >= rows) continue;
        const int req = first_req + (row_base + rho) / g;
        const int h = kvh * g + (row_base + rho) % g;
        const int64_t idx = ((int64_t)req * a.part.S + s) * a.Hq + h;
        float *op = a.part.o + idx * D;
#pragma unroll
        for (int db = 0; db < DB; db++) *(f32x4 *)(op + db * 16 + kq * 4) = oacc[db][nb];
        if (kq == 0) {
            a.part.ml[idx * 2] = m_run[nb];
            a.part.ml[idx * 2 + 1] = l;
        }
    }
}

}  // namespace

int launch_split_bf16(const SplitArgs &a, hipStream_t st) {
    if (a.n_sets == 0 || a.max_splits == 0) return SGL_OK;
    const int g = a.Hq / a.Hkv;
    int rows = (a.kind == 1 ? a.max_members : 1) * g;
    SplitArgs b = a;
    b.row_blocks = 1;
    if (rows > 64) {                 // big groups: several 64-row waves per group
        b.row_blocks = (rows + 63) / 64;
        rows = 64;
    }
    dim3 grid(a.Hkv, a.max_splits, a.n_sets * b.row_blocks), block(64);
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
#define SGL_LAUNCH(DD, NBB) \
    hipLaunchKernelGGL((split_bf16_kernel<DD, NBB>), grid, block, dyn, st, b)
    if (a.D == 128) {
        if (rows <= 16) SGL_LAUNCH(128, 1);
        else if (rows <= 32) SGL_LAUNCH(128, 2);
        else SGL_LAUNCH(128, 4);
    } else {
        if (rows <= 16) SGL_LAUNCH(64, 1);
        else if (rows <= 32) SGL_LAUNCH(64, 2);
        else SGL_LAUNCH(64, 4);
    }
#undef SGL_LAUNCH
    return hip_status(hipGetLastError());
}
