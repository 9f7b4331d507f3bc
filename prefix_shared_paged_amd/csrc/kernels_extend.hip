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
//   - the 4 waves gather the next tile's 64 K rows and 64 V rows of this KV
//     head by slot id straight from HBM into the other half of a
//     double-buffered LDS tile with global_load_lds_dwordx4 (no register
//     staging; the slot ids are fetched one tile ahead).  Such a load writes
//     LDS contiguously by lane, so each lane picks WHICH 16-byte chunk of its
//     row it fetches: chunk c of row r sits at position c ^ swz(r), an XOR
//     swizzle under which both the MFMA operand reads of K and the transposed
//     reads of V are bank-conflict free, with no padding;
//   - each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16_bf16 (keys on M, rows on N), so a lane owns one
//     query row's scores;
//   - online softmax in fp32 on raw scores: the scale is folded into the
//     exponent (one FMA per score), exponentials are v_exp_f32, the causal
//     mask is applied only on tiles that cross the diagonal, and the
//     accumulator is rescaled lazily -- only when a row's running maximum
//     grows by more than 2^8 (the exact result is unchanged: the stored
//     maximum is simply a slightly stale reference point);
//   - P is rounded to bf16 and O^T += V^T P^T runs on MFMA with V^T read by
//     ds_read_b64_tr_b16; the key order inside each MFMA matches the
//     accumulator layout of S^T, so P needs no lane exchange.
#include <type_traits>

#include "common.h"

namespace {

constexpr int BN = 64;        // keys per tile
constexpr int BM = 128;       // query rows per workgroup
constexpr int NT = 256;       // threads
constexpr float kLazy = 8.f;  // rescale only when the max grows by more than 2^8

// Position of 16-byte chunk c of LDS row r is c ^ swz<D>(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const void *p) {
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
    constexpr int ROWB = 2 * D;           // bytes per K or V row of one KV head
    constexpr int CHK = D / 8;            // 16-byte chunks per row
    constexpr int RPB = 64 / CHK;         // rows per 1 KiB direct-load block
    constexpr int NB = BN / RPB / 4;      // blocks per wave per tile (K and V each)
    constexpr int KTILE = BN * ROWB;
    constexpr int BUFB = 2 * KTILE;       // K tile then V tile
    // two separate LDS objects, one per buffer, so the compiler can tell that
    // reads of one buffer do not wait on the direct loads into the other
    __shared__ __attribute__((aligned(16))) unsigned char lds_buf0[BUFB];   // [K V]
    __shared__ __attribute__((aligned(16))) unsigned char lds_buf1[BUFB];   // [K V]

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
    const int E = (int)(q_off[r + 1] - t0);
    const int q0 = qt * tok_per_tile;                    // first new token of this tile
    if (q0 >= E) return;
    const int64_t rowi = req_rows[r];
    const int P = prefix_lens[r];
    if (rowi < 0 || rowi >= num_rows || P < 0) return;
    int kv_end = P + (q0 + tok_per_tile < E ? q0 + tok_per_tile : E);   // keys [0, kv_end)
    if (kv_end > stride) kv_end = (int)stride;
    const int32_t *row = r2t + rowi * stride;
    const int64_t rowstride_el = (int64_t)Hkv * D;

    // ---- this lane's query row ------------------------------------------------
    const int n32 = lane & 31, h2 = lane >> 5;
    const int rho = wave * 32 + n32;                 // row in the tile
    const int tok_local = q0 + rho / g;              // new-token index within the request
    const bool row_valid = tok_local < E;
    const int h = kvh * g + rho % g;
    const int pos = P + (row_valid ? tok_local : E - 1);   // absolute position
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
    float m_run = -INFINITY;     // reference maximum (log2 units of the scaled score)
    float l_run = 0.f;           // this lane's part of the row sum

    // ---- tile loader: wave w fills 1 KiB blocks w*NB .. w*NB+NB-1 of K and V --
    // lane -> (row r = block * RPB + lane / CHK, position lane % CHK), fetching
    // chunk (lane % CHK) ^ swz(r) of key tile0 + r.
    // Slot ids are loaded unconditionally (index clamped into the row) and
    // checked only when used; sl[b] holds the ids of the tile that goes into
    // LDS buffer b, so a load lands directly where its use reads it.
    int sl[2][NB];
    auto fetch_slots = [&](int tile0, int (&dst)[NB]) {
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int j = tile0 + (wave * NB + i) * RPB + lane / CHK;
            dst[i] = row[j < kv_end ? j : kv_end - 1];
        }
    };
    auto issue = [&](int buf, const int (&sl)[NB]) {
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int blk = wave * NB + i;
            const int rr = blk * RPB + lane / CHK;
            const int c = (lane % CHK) ^ swz<D>(rr);
            const int64_t off = (int64_t)safe_slot(sl[i], num_slots) * rowstride_el + kvh * D + c * 8;
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)(k_pool + off),
                                             (SGL_LDS void *)((buf ? lds_buf1 : lds_buf0) + blk * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)(v_pool + off),
                                             (SGL_LDS void *)((buf ? lds_buf1 : lds_buf0) + KTILE + blk * 1024), 16, 0,
                                             0);
        }
    };
    // V rows past the end of the context must hold zeros (their P is 0, and
    // whatever slot 0 holds must not turn 0 * v into NaN); runs after the
    // loads of that tile have landed.
    auto zero_tail = [&](int buf, int tile0) {
        const int nvalid = kv_end - tile0;
        if (nvalid >= BN) return;
        unsigned char *vt = (buf ? lds_buf1 : lds_buf0) + KTILE;
        for (int idx = tid; idx < (BN - nvalid) * CHK; idx += NT)
            *(uint4 *)(vt + (nvalid + idx / CHK) * ROWB + 16 * (idx % CHK)) = make_uint4(0, 0, 0, 0);
    };

    // Per-lane LDS byte offsets of the MFMA operand reads.  The swizzle of a
    // row depends only on bits that stay fixed across the 32-row K blocks and
    // the 16-row V steps, so the loop indices become immediate offsets.
    const int grp = (lane >> 4) & 1;                 // which 16 dims of a 32-dim block
    const int r4 = (lane & 15) >> 2, qq = lane & 3;
    int koff[QT];                                    // K operand of step t, key block 0
    {
        const int sk = swz<D>(n32);
#pragma unroll
        for (int t = 0; t < QT; t++) koff[t] = n32 * ROWB + 16 * ((2 * t + h2) ^ sk);
    }
    int voff0[DBLK], voff1[DBLK];                    // V^T reads of dim block b, PV step 0
    {
        const int v0 = 4 * h2 + r4, v1 = v0 + 8;
        const int s0 = swz<D>(v0), s1 = swz<D>(v1);
#pragma unroll
        for (int b = 0; b < DBLK; b++) {
            const int c = 4 * b + 2 * grp + (qq >> 1);
            voff0[b] = v0 * ROWB + 16 * (c ^ s0) + 8 * (qq & 1);
            voff1[b] = v1 * ROWB + 16 * (c ^ s1) + 8 * (qq & 1);
        }
    }

    // One 64-key tile from LDS buffer BUF.  Both 32-key blocks' S^T MFMAs are
    // issued first; block 0's softmax (VALU) then runs while block 1's S^T is in
    // the matrix pipe, and block 0's PV MFMAs while block 1's softmax runs.
    // MASK: the tile may cross the diagonal of some row.
    auto tile = [&](const int tile0, auto buf_tag, auto mask_tag) {
        constexpr int BUF = decltype(buf_tag)::value;
        constexpr bool MASK = decltype(mask_tag)::value;
        const unsigned char *Kt = BUF ? lds_buf1 : lds_buf0;
        const unsigned char *Vt = Kt + KTILE;
        // K operands of key block 0, read ahead of their MFMAs
        bf16x8 kf[QT];
#pragma unroll
        for (int t = 0; t < QT; t++) kf[t] = ld_bf16x8(Kt + koff[t]);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            // S^T = K Q^T (raw, unscaled scores) for keys kb*32 .. kb*32+31
#pragma unroll
            for (int j = 0; j < 16; j++) sacc[kb][j] = 0.f;
#pragma unroll
            for (int t = 0; t < QT; t++)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t], sacc[kb], 0, 0, 0);
            if (kb == 0) {
                // block 1's K operands are read while block 0's softmax and PV run
#pragma unroll
                for (int t = 0; t < QT; t++) kf[t] = ld_bf16x8(Kt + 32 * ROWB + koff[t]);
            }
            f32x16 sc = sacc[kb];
            if (MASK) {
                // key (tile-local) of accumulator element j: kb*32 + 8*(j/4) + 4*h2 + j%4
                const int lim = pos - tile0 - kb * 32 - 4 * h2;
#pragma unroll
                for (int j = 0; j < 16; j++)
                    if (8 * (j >> 2) + (j & 3) > lim) sc[j] = -INFINITY;
            }
            float mx = sc[0];
#pragma unroll
            for (int j = 1; j < 16; j++) mx = fmaxf(mx, sc[j]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_blk = mx * qscale;
            // lazy rescale: only when some row's maximum moved by more than 2^kLazy
            const bool need = m_blk > m_run + kLazy;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float m_new = need ? m_blk : m_run;
                const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < DBLK; b++) oacc[b] *= alpha;
                m_run = m_new;
            }
            // p = 2^(s * scale * log2e - m_run), rounded to bf16 for the PV product
            bf16x8 pf[2];        // B operands of the 2 PV steps of this block
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[j], qscale, -m_run));
                psum += p;
                pf[j >> 3][j & 7] = (__bf16)p;
            }
            l_run += psum;
            // O^T += V^T P^T; step st covers keys 16*st + {4*h2 + 0..3, 8 + 4*h2 + 0..3}
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++) {
                const int st = kb * 2 + s2;
#pragma unroll
                for (int b = 0; b < DBLK; b++) {
                    const unsigned char *p0 = Vt + st * 16 * ROWB + voff0[b];
                    const unsigned char *p1 = Vt + st * 16 * ROWB + voff1[b];
                    i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p0);
                    i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p1);
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    const i16x8 cat = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pf[s2],
                                                                     oacc[b], 0, 0, 0);
                }
            }
        }
    };

    const int n_tiles = (kv_end + BN - 1) / BN;
    const int min_pos = P + q0;                      // smallest position in the tile
    // tiles every row sees whole (no mask), rounded down to an even count so
    // both loops below start on LDS buffer 0
    const int n_full = min((min_pos + 1) / BN, n_tiles) & ~1;
    fetch_slots(0, sl[0]);
    issue(0, sl[0]);
    if (n_tiles > 1) fetch_slots(BN, sl[1]);
    wait_vm_all();
    zero_tail(0, 0);
    __syncthreads();
    // One tile: start loading tile it+1 into the other buffer, compute tile it,
    // then wait for the load and publish it.
    auto step = [&](const int it, auto buf_tag, auto mask_tag) {
        constexpr int BUF = decltype(buf_tag)::value;
        if (it + 1 < n_tiles) {
            if (it + 2 < n_tiles) fetch_slots((it + 2) * BN, sl[BUF]);   // before the direct loads
            issue(BUF ^ 1, sl[BUF ^ 1]);
        }
        tile(it * BN, buf_tag, mask_tag);
        wait_vm_all();
        if (it + 1 < n_tiles) zero_tail(BUF ^ 1, (it + 1) * BN);
        __syncthreads();
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    int it = 0;
    for (; it < n_full; it += 2) {                   // straight-line pairs, no mask
        step(it, B0{}, std::false_type{});
        step(it + 1, B1{}, std::false_type{});
    }
    for (; it + 1 < n_tiles; it += 2) {              // pairs that may cross the diagonal
        step(it, B0{}, std::true_type{});
        step(it + 1, B1{}, std::true_type{});
    }
    if (it < n_tiles) step(it, B0{}, std::true_type{});

    // ---- epilogue: normalise and store ----------------------------------------
    const float l = l_run + __shfl_xor(l_run, 32, 64);
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
    if (row_stride > 0x7fffffff) return SGL_ERR_UNSUPPORTED;   // positions are 32-bit in the kernel
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
