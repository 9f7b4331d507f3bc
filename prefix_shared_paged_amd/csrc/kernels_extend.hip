// kernels_extend.hip -- bf16 extend (prefix-aware prefill) attention for gfx950.
//
// The new tokens of a request attend causally to [cached prefix || new tokens]
// ("SGLang 深度拆解" (chenxutan.com) section 3.2 PagedPrefill: only the
// uncached tokens are computed, the whole context is read through the page
// table; "SGLang 深度解读" module 5: K/V rows are found through
// req_to_token).
//
// Work decomposition: one workgroup (4 waves) per (request, KV head, tile of
// 128 query rows).  A query row is a (new token, query head) pair; the g
// query heads that share the KV head are packed into the tile, so every K/V
// tile brought into LDS serves 128 rows.  Workgroup ids are ordered so that
// id % 8 (the XCD a workgroup lands on) follows the KV head: all tiles of one
// KV head share an XCD and its L2 holds that head's prefix.
//
// Per 64-key tile:
//   - 256 threads gather the 64 K rows and 64 V rows of this KV head by slot
//     id into registers (next tile, while the current one is computed) and
//     then into a double-buffered LDS tile (row-major, rows padded to 288 B
//     so MFMA operand reads and transposed reads are bank-conflict free);
//   - each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16_bf16 (keys on M, rows on N), so a lane owns one
//     query row's scores;
//   - online softmax in fp32 (running max / sum per row, rescale of the
//     accumulator), causal mask only on tiles that cross the diagonal;
//   - P is rounded to bf16 and O^T += V^T P^T runs on MFMA with V^T read by
//     ds_read_b64_tr_b16; the key order inside each MFMA matches the
//     accumulator layout of S^T, so P needs no lane exchange.
#include "common.h"

namespace {

constexpr int BN = 64;        // keys per tile
constexpr int BM = 128;       // query rows per workgroup
constexpr int ROWB = 288;     // padded LDS row (bytes) for D = 128
constexpr int NT = 256;       // threads

__device__ __forceinline__ bf16x8 ld_bf16x8(const void *p) {
    union { uint4 u; bf16x8 b; } x;
    x.u = *(const uint4 *)p;
    return x.b;
}
__device__ __forceinline__ bf16x8 lds_bf16x8(const unsigned char *p) {
    union { uint4 u; bf16x8 b; } x;
    x.u = *(const uint4 *)p;
    return x.b;
}

template <int D>
__global__ void __launch_bounds__(NT, 2) extend_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k_pool,
    const __bf16 *__restrict__ v_pool, int64_t num_slots, const int32_t *__restrict__ r2t,
    int64_t num_rows, int64_t stride, const int32_t *__restrict__ req_rows,
    const int32_t *__restrict__ prefix_lens, const int64_t *__restrict__ q_off, int Hq, int Hkv,
    int n_qtiles, float qscale, __bf16 *__restrict__ o, float *__restrict__ lse) {
    constexpr int QT = D / 16;            // k-steps of 16 dims for S^T
    constexpr int DBLK = D / 32;          // 32-dim output blocks
    constexpr int CH = D / 32;            // uint4 per thread per row part (4 threads per row)
    constexpr int TILEB = BN * ROWB;
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * TILEB];  // K0 V0 K1 V1

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int id = blockIdx.x;
    const int kvh = id % Hkv;
    const int rest = id / Hkv;
    const int qt = rest % n_qtiles;
    const int r = rest / n_qtiles;
    const int g = Hq / Hkv;
    const int tok_per_tile = BM / g;

    const int64_t t0 = q_off[r];
    const int64_t E = q_off[r + 1] - t0;
    const int64_t q0 = (int64_t)qt * tok_per_tile;       // first new token of this tile
    if (q0 >= E) return;
    const int64_t rowi = req_rows[r];
    const int64_t P = prefix_lens[r];
    if (rowi < 0 || rowi >= num_rows || P < 0) return;
    int64_t kv_end = P + (q0 + tok_per_tile < E ? q0 + tok_per_tile : E);   // keys [0, kv_end)
    if (kv_end > stride) kv_end = stride;
    const int32_t *row = r2t + rowi * stride;
    const int64_t rowstride_el = (int64_t)Hkv * D;

    // ---- this lane's query row ------------------------------------------------
    const int n32 = lane & 31, h2 = lane >> 5;
    const int rho = wave * 32 + n32;                 // row in the tile
    const int64_t tok_local = q0 + rho / g;          // new-token index within the request
    const bool row_valid = tok_local < E;
    const int h = kvh * g + rho % g;
    const int64_t pos = P + (row_valid ? tok_local : E - 1);   // absolute position
    bf16x8 qf[QT];
    {
        const __bf16 *src = q + ((t0 + (row_valid ? tok_local : 0)) * Hq + h) * D + 8 * h2;
#pragma unroll
        for (int t = 0; t < QT; t++) qf[t] = ld_bf16x8(src + 16 * t);
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; b++)
#pragma unroll
        for (int j = 0; j < 16; j++) oacc[b][j] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // ---- tile loader: thread -> (key = tid / 4, quarter = tid % 4) -------------
    const int ld_key = tid >> 2, ld_part = tid & 3;
    uint4 kreg[CH], vreg[CH];
    auto gather = [&](int64_t tile0) {
        const int64_t j = tile0 + ld_key;
        if (j < kv_end) {
            const int64_t s = safe_slot(row[j], num_slots);
            const uint4 *ks = (const uint4 *)(k_pool + s * rowstride_el + kvh * D + ld_part * (D / 4));
            const uint4 *vs = (const uint4 *)(v_pool + s * rowstride_el + kvh * D + ld_part * (D / 4));
#pragma unroll
            for (int c = 0; c < CH; c++) { kreg[c] = ks[c]; vreg[c] = vs[c]; }
        } else {
#pragma unroll
            for (int c = 0; c < CH; c++) { kreg[c] = make_uint4(0, 0, 0, 0); vreg[c] = make_uint4(0, 0, 0, 0); }
        }
    };
    auto stash = [&](int buf) {
        unsigned char *kd = lds + buf * 2 * TILEB + ld_key * ROWB + ld_part * (D / 2);
        unsigned char *vd = kd + TILEB;
#pragma unroll
        for (int c = 0; c < CH; c++) {
            *(uint4 *)(kd + 16 * c) = kreg[c];
            *(uint4 *)(vd + 16 * c) = vreg[c];
        }
    };

    const int n_tiles = (int)ceil_div64(kv_end, BN);
    const int64_t min_pos = P + q0;                 // smallest position in the tile
    gather(0);
    stash(0);
    __syncthreads();

    for (int it = 0; it < n_tiles; it++) {
        const int buf = it & 1;
        const int64_t tile0 = (int64_t)it * BN;
        if (it + 1 < n_tiles) gather(tile0 + BN);
        const unsigned char *Kt = lds + buf * 2 * TILEB;
        const unsigned char *Vt = Kt + TILEB;

        // ---- S^T = K Q^T for two 32-key blocks -----------------------------------
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            f32x16 c;
#pragma unroll
            for (int j = 0; j < 16; j++) c[j] = 0.f;
            const unsigned char *kr = Kt + (kb * 32 + n32) * ROWB + 16 * h2;
#pragma unroll
            for (int t = 0; t < QT; t++)
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_bf16x8(kr + 32 * t), qf[t], c, 0, 0, 0);
            sacc[kb] = c;
        }

        // ---- online softmax for this lane's row ------------------------------------
        const bool diag = tile0 + BN - 1 > min_pos;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int j = 0; j < 16; j++) {
                float x = sacc[kb][j] * qscale;
                if (diag) {
                    const int64_t key = tile0 + kb * 32 + 8 * (j >> 2) + 4 * h2 + (j & 3);
                    x = key <= pos ? x : -INFINITY;
                }
                sacc[kb][j] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.f;
        bf16x8 pf[4];                      // B operands of the 4 PV steps (16 keys each)
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const float p = exp2f(sacc[kb][j] - m_new);
                psum += p;
                pf[kb * 2 + (j >> 3)][j & 7] = (__bf16)p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < DBLK; b++) oacc[b] *= alpha;

        // ---- O^T += V^T P^T ------------------------------------------------------
        // step st covers keys 16*st + {4*h2 + 0..3, 8 + 4*h2 + 0..3} (per lane half).
        const int grp = (lane >> 4) & 1;             // which 16 dims of a 32-dim block
        const int r4 = (lane & 15) >> 2, qq = lane & 3;
#pragma unroll
        for (int st = 0; st < 4; st++) {
#pragma unroll
            for (int b = 0; b < DBLK; b++) {
                const int col = (b * 32 + grp * 16 + qq * 4) * 2;
                const unsigned char *p0 = Vt + (16 * st + 4 * h2 + r4) * ROWB + col;
                const unsigned char *p1 = p0 + 8 * ROWB;
                i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p0);
                i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p1);
                union { i16x4 hh[2]; bf16x8 bb; } va;
                va.hh[0] = lo4;
                va.hh[1] = hi4;
                oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va.bb, pf[st], oacc[b], 0, 0, 0);
            }
        }

        if (it + 1 < n_tiles) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: normalise and store ----------------------------------------
    float l = l_run + __shfl_xor(l_run, 32, 64);
    if (!row_valid) return;
    const float inv = 1.f / l;
    __bf16 *dst = o + ((t0 + tok_local) * Hq + h) * D;
#pragma unroll
    for (int b = 0; b < DBLK; b++)
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] = (__bf16)(oacc[b][a4 * 4 + e] * inv);
            *(bf16x4 *)(dst + b * 32 + 8 * a4 + 4 * h2) = v;
        }
    if (lse && h2 == 0) lse[(t0 + tok_local) * Hq + h] = (m_run + log2f(l)) * kLn2;
}

}  // namespace

int launch_extend_bf16(const __bf16 *q, const __bf16 *k_pool, const __bf16 *v_pool,
                       int64_t num_slots, const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                       const int32_t *req_rows, const int32_t *prefix_lens, const int64_t *q_off,
                       int32_t batch, int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D,
                       float scale, __bf16 *o, float *lse, hipStream_t st) {
    if (batch == 0 || max_extend_len == 0) return SGL_OK;
    const int g = Hq / Hkv;
    const int tok_per_tile = BM / g;
    const int n_qtiles = (int)ceil_div64(max_extend_len, tok_per_tile);
    const int64_t n_wg = (int64_t)n_qtiles * batch * Hkv;
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const float qs = scale * kLog2e;
    if (D == 128)
        hipLaunchKernelGGL(extend_bf16_kernel<128>, dim3((unsigned)n_wg), dim3(NT), 0, st, q, k_pool,
                           v_pool, num_slots, r2t, num_rows, row_stride, req_rows, prefix_lens, q_off,
                           Hq, Hkv, n_qtiles, qs, o, lse);
    else
        hipLaunchKernelGGL(extend_bf16_kernel<64>, dim3((unsigned)n_wg), dim3(NT), 0, st, q, k_pool,
                           v_pool, num_slots, r2t, num_rows, row_stride, req_rows, prefix_lens, q_off,
                           Hq, Hkv, n_qtiles, qs, o, lse);
    return hip_status(hipGetLastError());
}
