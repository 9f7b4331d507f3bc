// kernels_mla.hip -- split-K decode over a latent KV cache (MLA-style).
//
// DeepSeek's MLA attention, with the decompression matrices absorbed into the
// query and output projections, runs directly on the compressed latent: one
// KV "head" per token of Dqk = 576 dims (512 compressed K/V dims + 64 RoPE
// dims), scores over all 576, values over the first 512, shared by every
// query head ("Lecture 16 · 案例研究：SGLang" (semidirectx.com) section 4).  So
// it is grouped-query attention with one KV head, g = Hq, and K and V read
// from the same rows: a token's latent is read once for both contractions.
//
// Layout: latent pool [num_slots, 576] bf16 (1152 bytes per token); q [.., Hq,
// 576]; o [.., Hq, 512].  Work item (as in kernels_decode.hip): a split of
// keys of a request (flat, suffix) or of a group's shared prefix (cascade),
// and a block of 16-row query blocks (request x head).  Two kernels:
//   split_mla_full_kernel (flat and suffix splits, every Hq): one wave per
//     16-row block over all 576 score dims and all 512 value dims, no
//     reduction across waves; the waves of a workgroup (1, 2 or 4 row blocks)
//     share each 16-key latent tile (18 KiB) in LDS, gathered by slot with
//     non-temporal direct loads into a ring of 2 (one or two blocks: four
//     workgroups per CU) or 4 tiles (four blocks, whose value contraction
//     takes the tiles in pairs);
//   split_mla_kernel (the cascade's prefix stage, up to 4 blocks): every
//     16-row block gets four waves: wave q computes the partial S^T = K Q^T
//     of the block over its share of the 576 score dims (5, 5, 4, 4 MFMA
//     steps of 32), the four partial tiles are summed through LDS, and each
//     wave then runs the softmax and O^T += V^T P^T for its quarter of the
//     512 value dims -- so a wave holds a fifth of Q and a quarter of O; two
//     tiles in flight.
#include <utility>

#include "common.h"
#include "decode_util.h"

namespace {

using namespace sgl_decode;

constexpr int MT = 16;          // keys per tile
constexpr int DQK = 576;        // score dims
constexpr int DV = 512;         // value dims
constexpr int RB = DQK * 2;     // bytes per latent row
constexpr int TBM = MT * RB;    // bytes per tile (18 KiB)
constexpr int NIM = TBM / 1024; // 1 KiB direct-load instructions per tile (18)
constexpr int MLA_DEPTH = 2;

// Position of 16-byte chunk c of tile row r is c ^ msw(r), an XOR inside the
// row's aligned groups of 8 chunks (72 chunks per row = 9 groups).  Rows are
// 1152 bytes apart, so row r starts in the (r % 2) half of a 256-byte bank
// line.  msw maps the eight rows of each parity to distinct chunk positions
// (K operand reads: 16 rows, one chunk each, fall on 16 distinct 16-byte
// bank groups), and rows 2j and 2j + 2 land on different chunk pairs (V^T
// reads: a half wave reads two adjacent chunks of each of 8 consecutive rows,
// 256 bytes on distinct banks).
__device__ __forceinline__ int msw(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

// RBW 16-row blocks per workgroup, four waves each
template <int RBW>
__global__ void __launch_bounds__(256 * RBW) split_mla_kernel(SplitArgs a) {
    constexpr int NW = 4 * RBW;                    // waves per workgroup
    constexpr int QS = 5;                          // MFMA k-steps of 32 dims per wave (at most)
    constexpr int DBW = DV / 4 / 16;               // 8 16-dim output blocks per wave
    __shared__ __attribute__((aligned(16))) unsigned char t_lds[MLA_DEPTH * TBM];
    __shared__ __attribute__((aligned(16))) f32x4 s_part[RBW][4][64];   // partial S^T tiles
    extern __shared__ int32_t slot_lds[];          // [chunk]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rbw = w >> 2, quarter = w & 3;       // row block in the workgroup, dim quarter
    const int t_lo = quarter * 5 - (quarter > 2 ? quarter - 2 : 0);   // first S^T step: 0, 5, 10, 14
    const int n_st = quarter < 2 ? 5 : 4;          // S^T steps of this wave
    auto wg_barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- work item: set, split, rows (uniform over the workgroup) --------------
    const int n_rbg = (a.row_blocks + RBW - 1) / RBW;
    const int id = blockIdx.x;
    const int rbg = id % n_rbg;
    const int64_t item = id / n_rbg;               // = split * n_sets + set
    const int set = (int)(item % a.n_sets);
    const int s = (int)(item / a.n_sets);
    if (s >= a.max_splits) return;
    const int g = a.Hq;
    int first_req, n_members;
    int64_t lo, hi, ref_row;
    if (a.kind == 1) {
        first_req = a.group_ptr[set];
        n_members = a.group_ptr[set + 1] - first_req;
        if (n_members <= 0 || first_req < 0 || first_req + n_members > a.batch) return;
        const int64_t P = a.group_prefix_len[set];
        lo = 0;
        hi = P < 0 ? 0 : P;
        ref_row = a.req_rows[first_req];
    } else {
        first_req = set;
        n_members = 1;
        const int64_t L = a.seq_lens[set];
        ref_row = a.req_rows[set];
        lo = 0;
        if (a.kind == 2) {
            const int grp = wave_find_group(a.group_ptr, a.G, set);
            const int64_t P = a.group_prefix_len[grp];
            lo = P < 0 ? 0 : (P > L ? L : P);
        }
        hi = L;
    }
    if (n_members * g <= rbg * RBW * 16) return;
    if (ref_row < 0 || ref_row >= a.num_rows) return;
    if (hi > a.row_stride) hi = a.row_stride;
    const int64_t n_split = ceil_div64(hi - lo, a.chunk);
    if (s >= n_split || s >= a.part.S) return;
    const int64_t k0 = lo + (int64_t)s * a.chunk;
    const int nk = (int)((k0 + a.chunk < hi ? k0 + a.chunk : hi) - k0);
    const int N = (nk + MT - 1) / MT;
    const int row_base = (rbg * RBW + rbw) * 16;   // first query row of this wave's block
    const int rows = n_members * g - row_base;     // may be <= 0: the wave still loads

    const int32_t *row = a.r2t + ref_row * a.row_stride + k0;
    for (int j = threadIdx.x; j < nk; j += 64 * NW) slot_lds[j] = safe_slot(row[j], a.num_slots);

    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand of this wave's steps: lane (row n16, kq) holds dims
    // 32(t_lo + t) + 8kq + i in step t
    bf16x8 qf[QS];
    {
        const int rho = n16 < rows ? n16 : 0;
        const int rr = row_base + rho < n_members * g ? row_base + rho : 0;
        const __bf16 *src = (const __bf16 *)a.q + ((int64_t)(first_req + rr / g) * a.Hq + rr % g) * DQK +
                            32 * t_lo + 8 * kq;
#pragma unroll
        for (int t = 0; t < QS; t++) qf[t] = t < n_st ? ld_q(src + 32 * t) : bf16x8{};
        if (n16 >= rows)
#pragma unroll
            for (int t = 0; t < QS; t++) qf[t] = bf16x8{};
    }

    // ---- direct loads: instruction ii covers tile bytes [1024 ii, 1024 ii + 1024);
    // wave w issues ii = w, w + NW, ... (the first NIM % NW waves one more)
    constexpr int MAXI = (NIM + NW - 1) / NW;
    int lrow[MAXI], lsrc[MAXI];
#pragma unroll
    for (int u = 0; u < MAXI; u++) {
        const int ii = w + NW * u;
        const int off = (ii < NIM ? ii : 0) * 1024 + 16 * lane;
        lrow[u] = off / RB;
        const int c = (off % RB) / 16;
        lsrc[u] = 16 * (c ^ msw(lrow[u]));
    }
    const int n_mine = (NIM - w + NW - 1) / NW;    // instructions this wave issues per tile
    const char *pool = (const char *)a.k_pool;

    __syncthreads();   // slot table visible

    auto issue = [&](int n, unsigned char *dst) {
#pragma unroll
        for (int u = 0; u < MAXI; u++) {
            if (u < n_mine) {
                const int kk = min(n * MT + lrow[u], nk - 1);
                const char *src = pool + (int64_t)slot_lds[kk] * RB + lsrc[u];
                __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                                 (SGL_LDS void *)(dst + (w + NW * u) * 1024), 16, 0, 2 /* nt */);
            }
        }
    };
    // byte offset of chunk c of tile row r
    auto at = [&](int r, int c) { return r * RB + 16 * (c ^ msw(r)); };

    f32x4 oacc[DBW];
#pragma unroll
    for (int db = 0; db < DBW; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float qscale = a.scale * kLog2e;
    // K operand of step t: lane (key n16, kq) reads chunk 4t + kq of row n16
    // V^T of 16-dim block db of this quarter: lane (r4, qq) of group kq reads 4
    // dims of row 4kq + r4; the result gives lane (dim, kq) keys 4kq .. 4kq+3
    const int r4 = n16 >> 2, qq = n16 & 3;
    const int vr = kq * 4 + r4;

    auto tile = [&](int n, const unsigned char *tb) {
        const uint32_t base = lds_addr(tb);
        // partial S^T over this wave's dims (the 5th step of a 4-step wave reads
        // a real chunk and multiplies it by a zero Q operand)
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        {
            uint32_t ad[QS];
#pragma unroll
            for (int t = 0; t < QS; t++) ad[t] = base + at(n16, 4 * min(t_lo + t, DQK / 32 - 1) + kq);
            u32x4 raw[QS];
            lds_read_raw128(raw, ad);
#pragma unroll
            for (int t = 0; t < QS; t++)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, raw[t]), qf[t], sacc, 0, 0,
                                                               0);
        }
        // sum the row block's four partial tiles
        s_part[rbw][quarter][lane] = sacc;
        lgkm_wait0();
        wg_barrier();
        sacc = s_part[rbw][0][lane] + s_part[rbw][1][lane] + s_part[rbw][2][lane] + s_part[rbw][3][lane];
        // online softmax (lazy reference maximum, as in kernels_decode.hip)
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float x = n * MT + kq * 4 + j < nk ? sacc[j] * qscale : -INFINITY;
            sv[j] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool move = mx > m_run + 8.f;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DBW; db++) oacc[db] *= alpha;
            m_run = m_new;
        }
        bf16x4 pf;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float pj = __builtin_amdgcn_exp2f(sv[j] - m_run);
            l_run += pj;
            pf[j] = (__bf16)pj;
        }
        uint32_t ad[DBW];
#pragma unroll
        for (int db = 0; db < DBW; db++)
            ad[db] = base + at(vr, quarter * 16 + 2 * db + (qq >> 1)) + 8 * (qq & 1);
        i16x4 vt[DBW];
        lds_read_tr16(vt, ad);
#pragma unroll
        for (int db = 0; db < DBW; db++)
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[db], __builtin_bit_cast(i16x4, pf), oacc[db],
                                                                 0, 0, 0);
    };

    // ring of MLA_DEPTH tiles: this wave's loads of tile n have landed when
    // only the later tile's remain (their count is this wave's n_mine)
    for (int t = 0; t < MLA_DEPTH && t < N; t++) issue(t, t_lds + (t % MLA_DEPTH) * TBM);
    for (int n = 0; n < N; n++) {
        if (n + 1 < N) {
            if (n_mine == 5) vm_wait<5>();
            else if (n_mine == 4) vm_wait<4>();
            else if (n_mine == 3) vm_wait<3>();
            else if (n_mine == 2) vm_wait<2>();
            else if (n_mine == 1) vm_wait<1>();
            else vm_wait<0>();
        } else {
            vm_wait<0>();
        }
        wg_barrier();
        unsigned char *tb = t_lds + (n % MLA_DEPTH) * TBM;
        tile(n, tb);
        if (n + MLA_DEPTH < N) {
            lgkm_wait0();
            wg_barrier();                              // every wave is done with this buffer
            issue(n + MLA_DEPTH, tb);
        }
    }

    // ---- the split's state: (m, l) by quarter 0, o by every quarter ------------
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 >= rows) return;
    const int rr = row_base + n16;
    const int req = first_req + rr / g;
    const int h = rr % g;
    const int64_t idx = ((int64_t)req * a.part.S + s) * a.Hq + h;
    float *op = a.part.o + idx * DV + quarter * (DV / 4);
#pragma unroll
    for (int db = 0; db < DBW; db++) *(f32x4 *)(op + db * 16 + kq * 4) = oacc[db];
    if (quarter == 0 && kq == 0) *(float2 *)(a.part.ml + idx * 2) = make_float2(m_run, l);
}

// Immediate-offset LDS reads (inline asm for the reason given in
// decode_util.h); OFF is a byte offset added to the address.
template <int OFF>
__device__ __forceinline__ void ds_b128(u32x4 &r, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr16(i32x2 &r, uint32_t addr) {
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
// s_waitcnt vmcnt(n) for a wave-uniform n <= M
template <int M>
__device__ __forceinline__ void vm_wait_upto(int n) {
    if constexpr (M == 0) {
        vm_wait<0>();
    } else {
        if (n >= M) vm_wait<M>();
        else vm_wait_upto<M - 1>(n);
    }
}
// maximum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max_across_kq(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
template <class F, int... I>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F &&f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// One wave per 16-row block over all 576 score dims and all 512 value dims:
// no reduction across waves.  The RBW waves of a workgroup (RBW row blocks)
// share each latent tile; a ring of DEPTH tiles lets one barrier per tile
// both publish the tile's direct loads and retire the buffer they refill.
// Four blocks take a ring of four (72 KiB, two workgroups per CU) and run the
// value contraction over pairs of tiles (32 keys per 16x16x32 MFMA); one or
// two blocks a ring of two (36 KiB: four workgroups per CU keep more rows in
// flight than a deeper ring would) and 16-key steps.  A wave keeps its
// block's Q operand (72 VGPRs) and O^T accumulators (128); with four or two
// blocks the kernel fits 256 VGPRs, two waves per SIMD.  SHARED: an item
// (request, split) has several row-block groups, which then read each tile
// through the same XCD's L2.
template <int RBW, int DEPTH, bool SHARED>
__global__ void __launch_bounds__(64 * RBW, DEPTH >= 4 ? 2 : 1) split_mla_full_kernel(SplitArgs a) {
    constexpr int QS = DQK / 32;                   // 18 S^T steps
    constexpr int DB = DV / 16;                    // 32 output blocks of 16 dims
    constexpr int KB = 3;                          // K operand reads per batch
    constexpr int VB = 8;                          // V^T reads per batch
    constexpr int TPS = DEPTH >= 4 ? 2 : 1;        // tiles per O^T step
    constexpr int VB2 = 4;                         // output blocks per batch of paired V^T reads
    __shared__ __attribute__((aligned(16))) unsigned char t_lds[DEPTH * TBM];
    extern __shared__ int32_t slot_lds[];          // [chunk]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work item (as split_mla_kernel, ids ordered as below) --------------------
    const int n_rbg = (a.row_blocks + RBW - 1) / RBW;
    const int id = blockIdx.x;
    // SHARED (several row-block groups per item): the groups of one item sit
    // 8 ids apart, on the same XCD and dispatched together, so the later
    // groups' tile loads find the first group's in that XCD's L2 (the grid is
    // a multiple of 8 * n_rbg; ids past the last item exit below)
    const int rbg = SHARED ? (id / 8) % n_rbg : id % n_rbg;
    const int64_t item = SHARED ? (int64_t)(id / (8 * n_rbg)) * 8 + id % 8 : id / n_rbg;
    const int set = (int)(item % a.n_sets);
    const int s = (int)(item / a.n_sets);
    if (s >= a.max_splits) return;
    const int g = a.Hq;
    int first_req, n_members;
    int64_t lo, hi, ref_row;
    if (a.kind == 1) {
        first_req = a.group_ptr[set];
        n_members = a.group_ptr[set + 1] - first_req;
        if (n_members <= 0 || first_req < 0 || first_req + n_members > a.batch) return;
        const int64_t P = a.group_prefix_len[set];
        lo = 0;
        hi = P < 0 ? 0 : P;
        ref_row = a.req_rows[first_req];
    } else {
        first_req = set;
        n_members = 1;
        const int64_t L = a.seq_lens[set];
        ref_row = a.req_rows[set];
        lo = 0;
        if (a.kind == 2) {
            const int grp = wave_find_group(a.group_ptr, a.G, set);
            const int64_t P = a.group_prefix_len[grp];
            lo = P < 0 ? 0 : (P > L ? L : P);
        }
        hi = L;
    }
    if (n_members * g <= rbg * RBW * 16) return;
    if (ref_row < 0 || ref_row >= a.num_rows) return;
    if (hi > a.row_stride) hi = a.row_stride;
    const int64_t n_split = ceil_div64(hi - lo, a.chunk);
    if (s >= n_split || s >= a.part.S) return;
    const int64_t k0 = lo + (int64_t)s * a.chunk;
    const int nk = (int)((k0 + a.chunk < hi ? k0 + a.chunk : hi) - k0);
    const int N = (nk + MT - 1) / MT;
    const int row_base = (rbg * RBW + w) * 16;
    const int rows = n_members * g - row_base;     // may be <= 0: the wave still loads

    const int32_t *row = a.r2t + ref_row * a.row_stride + k0;
    for (int j = threadIdx.x; j < nk; j += 64 * RBW) slot_lds[j] = safe_slot(row[j], a.num_slots);

    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand: lane (row n16, kq) holds dims 32t + 8kq + i in step t --------
    bf16x8 qf[QS];
    {
        const int rho = n16 < rows ? n16 : 0;
        const int rr = row_base + rho < n_members * g ? row_base + rho : 0;
        const __bf16 *src = (const __bf16 *)a.q + ((int64_t)(first_req + rr / g) * a.Hq + rr % g) * DQK + 8 * kq;
#pragma unroll
        for (int t = 0; t < QS; t++) qf[t] = n16 < rows ? ld_q(src + 32 * t) : bf16x8{};
    }

    // ---- direct loads: instruction ii covers tile bytes [1024 ii, 1024 ii + 1024);
    // wave w issues ii = w, w + RBW, ...
    constexpr int MAXI = (NIM + RBW - 1) / RBW;
    const int n_mine = (NIM - w + RBW - 1) / RBW;
    const char *pool = (const char *)a.k_pool;

    __syncthreads();   // slot table visible

    auto issue = [&](int n, unsigned char *dst) {
        // tile row and source byte offset of each of this lane's pieces;
        // with several waves (two per SIMD) they are recomputed per tile from
        // a lane id the compiler cannot see through, since kept live across
        // the loop they would cost registers the MFMA operands need
        int ln = lane;
        if constexpr (RBW > 1) asm volatile("" : "+v"(ln));
        int lrow[MAXI], lsrc[MAXI];
#pragma unroll
        for (int u = 0; u < MAXI; u++) {
            const int ii = w + RBW * u;
            const int off = (ii < NIM ? ii : 0) * 1024 + 16 * ln;
            lrow[u] = off / RB;
            lsrc[u] = 16 * ((off % RB) / 16 ^ msw(lrow[u]));
        }
        int32_t sl[MAXI];                          // all look-ups first: one LDS wait
#pragma unroll
        for (int u = 0; u < MAXI; u++) sl[u] = slot_lds[min(n * MT + lrow[u], nk - 1)];
#pragma unroll
        for (int u = 0; u < MAXI; u++) {
            if (u < n_mine) {
                const char *src = pool + (int64_t)sl[u] * RB + lsrc[u];
                // tiles that another row-block group reads too stay in L2;
                // otherwise non-temporal
                __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                                 (SGL_LDS void *)(dst + (w + RBW * u) * 1024), 16, 0,
                                                 SHARED ? 0 : 2 /* nt */);
            }
        }
    };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float qscale = a.scale * kLog2e;
    // K operand of step t: chunk 4t + kq of row n16, at position (4t + kq) ^ msw
    // inside its group of 8: base (t even / odd) + 128 (t / 2)
    const int mk = msw(n16);
    const uint32_t koff0 = n16 * RB + 16 * ((0 + kq) ^ mk);
    const uint32_t koff1 = n16 * RB + 16 * ((4 + kq) ^ mk);
    // V^T of output block db: lane (r4, qq) of group kq reads dims 16 db + 4 qq ..
    // of row 4kq + r4: chunk 2db + (qq >> 1), byte 8 (qq & 1); for db = 4j + d
    // the position is 8j + ((2d + (qq >> 1)) ^ msw(row)): base (d) + 128 j
    const int r4 = n16 >> 2, qq = n16 & 3;
    const int vr = kq * 4 + r4;
    const int mv = msw(vr);
    uint32_t voff[4];
#pragma unroll
    for (int d = 0; d < 4; d++) voff[d] = vr * RB + 16 * ((2 * d + (qq >> 1)) ^ mv) + 8 * (qq & 1);

    // S^T of one 16-key tile (KB independent accumulators: step t feeds t % KB,
    // so consecutive MFMAs do not wait on each other)
    auto scores = [&](uint32_t base) -> f32x4 {
        const uint32_t kb0 = base + koff0, kb1 = base + koff1;
        f32x4 sp[KB];
#pragma unroll
        for (int i = 0; i < KB; i++) sp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        static_for(std::make_integer_sequence<int, QS / KB>{}, [&](auto bi) {
            constexpr int B0 = decltype(bi)::value * KB;
            u32x4 raw[KB];
            static_for(std::make_integer_sequence<int, KB>{}, [&](auto ti) {
                constexpr int T = B0 + decltype(ti)::value;
                ds_b128<128 * (T >> 1)>(raw[decltype(ti)::value], (T & 1) ? kb1 : kb0);
            });
            lgkm_wait_tied(raw);
#pragma unroll
            for (int i = 0; i < KB; i++)
                sp[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, raw[i]), qf[B0 + i], sp[i],
                                                                0, 0, 0);
        });
        f32x4 sacc = sp[0];
#pragma unroll
        for (int i = 1; i < KB; i++) sacc += sp[i];
        return sacc;
    };
    // online softmax over NT * 16 keys from tile n0 on (lazy reference
    // maximum); p[4 t + j] is key 16 (n0 + t) + 4 kq + j of row n16
    auto softmax = [&](int n0, const f32x4 (&s)[TPS], float (&p)[4 * TPS]) {
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < TPS; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = (n0 + t) * MT + kq * 4 + j < nk ? s[t][j] * qscale : -INFINITY;
                p[4 * t + j] = x;
                mx = fmaxf(mx, x);
            }
        mx = max_across_kq(mx);
        const bool move = mx > m_run + 8.f;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
            m_run = m_new;
        }
#pragma unroll
        for (int j = 0; j < 4 * TPS; j++) {
            p[j] = __builtin_amdgcn_exp2f(p[j] - m_run);
            l_run += p[j];
        }
    };

    if constexpr (TPS == 1) {
        // one tile per step: O^T += V^T P^T over its 16 keys (16x16x16 MFMAs)
        auto tile = [&](int n, const unsigned char *tb) {
            const uint32_t base = lds_addr(tb);
            const f32x4 s[1] = {scores(base)};
            float p[4];
            softmax(n, s, p);
            bf16x4 pf;
#pragma unroll
            for (int j = 0; j < 4; j++) pf[j] = (__bf16)p[j];
            const i16x4 pb = __builtin_bit_cast(i16x4, pf);
            static_for(std::make_integer_sequence<int, DB / VB>{}, [&](auto bi) {
                constexpr int D0 = decltype(bi)::value * VB;
                i32x2 vt[VB];
                static_for(std::make_integer_sequence<int, VB>{}, [&](auto di) {
                    constexpr int DBI = D0 + decltype(di)::value;
                    ds_tr16<128 * (DBI >> 2)>(vt[decltype(di)::value], base + voff[DBI & 3]);
                });
                lgkm_wait_tied(vt);
#pragma unroll
                for (int i = 0; i < VB; i++)
                    oacc[D0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vt[i]), pb,
                                                                             oacc[D0 + i], 0, 0, 0);
            });
        };
        // ring of DEPTH tiles, DEPTH - 1 in flight: at the top of step n this
        // wave's loads of tile n have landed when only those of tiles n+1 ..
        // n+DEPTH-2 remain; after the barrier every wave has also finished tile
        // n-1, whose buffer takes tile n+DEPTH-1
        for (int t = 0; t < DEPTH - 1 && t < N; t++) issue(t, t_lds + t * TBM);
        for (int n = 0; n < N; n++) {
            const int later = min(DEPTH - 2, N - 1 - n);
            vm_wait_upto<MAXI * (DEPTH - 2)>(n_mine * later);
            lgkm_wait0();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (n + DEPTH - 1 < N) issue(n + DEPTH - 1, t_lds + ((n + DEPTH - 1) % DEPTH) * TBM);
            tile(n, t_lds + (n % DEPTH) * TBM);
        }
    } else {
        // tiles in pairs: the scores of an even tile are kept until the next
        // (odd) tile's, then one softmax covers both and O^T += V^T P^T runs
        // over their 32 keys with 16x16x32 MFMAs (half the instructions of
        // two 16-key steps).  Contraction slot 8 kq + j of a lane is key
        // 4 kq + j of the even tile for j < 4 and key 4 kq + j - 4 of the odd
        // one: the V^T operand is the two tiles' transposed reads side by
        // side, the P^T operand the two score fragments.  With no odd tile
        // (N odd) the even tile's buffer stands in for it under zero weights.
        auto pair = [&](int n0, const f32x4 &sa, uint32_t ba, const f32x4 &sb, uint32_t bb) {
            const f32x4 s[2] = {sa, sb};
            float p[8];
            softmax(n0, s, p);
            bf16x8 pb;
#pragma unroll
            for (int j = 0; j < 8; j++) pb[j] = (__bf16)p[j];
            static_for(std::make_integer_sequence<int, DB / VB2>{}, [&](auto bi) {
                constexpr int D0 = decltype(bi)::value * VB2;
                i32x2 vt[2 * VB2];
                static_for(std::make_integer_sequence<int, VB2>{}, [&](auto di) {
                    constexpr int DBI = D0 + decltype(di)::value;
                    ds_tr16<128 * (DBI >> 2)>(vt[2 * decltype(di)::value], ba + voff[DBI & 3]);
                    ds_tr16<128 * (DBI >> 2)>(vt[2 * decltype(di)::value + 1], bb + voff[DBI & 3]);
                });
                lgkm_wait_tied(vt);
#pragma unroll
                for (int i = 0; i < VB2; i++) {
                    const u32x4 v = {(unsigned)vt[2 * i][0], (unsigned)vt[2 * i][1], (unsigned)vt[2 * i + 1][0],
                                     (unsigned)vt[2 * i + 1][1]};
                    oacc[D0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb,
                                                                           oacc[D0 + i], 0, 0, 0);
                }
            });
        };
        // ring of DEPTH tiles, F = DEPTH - 2 in flight: at the top of step n
        // this wave's loads of tile n have landed when only those of tiles
        // n+1 .. n+F-1 remain; after the barrier every wave is past step
        // n-1, so tile n-2 (scored at step n-2, its values read by step n-1
        // at the latest) is done and its buffer takes tile n+F, while tile
        // n-1 (still to be read when n is odd) keeps its own.
        constexpr int F = DEPTH - 2;
        static_assert(F >= 2, "pairs of tiles take a ring of four or more");
        for (int t = 0; t < F && t < N; t++) issue(t, t_lds + t * TBM);
        f32x4 s_even = f32x4{0.f, 0.f, 0.f, 0.f};
        uint32_t b_even = lds_addr(t_lds);
        for (int n = 0; n < N; n++) {
            vm_wait_upto<MAXI * (F - 1)>(n_mine * min(F - 1, N - 1 - n));
            lgkm_wait0();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (n + F < N) issue(n + F, t_lds + ((n + F) % DEPTH) * TBM);
            const uint32_t base = lds_addr(t_lds + (n % DEPTH) * TBM);
            const f32x4 s = scores(base);
            if (n & 1) {
                pair(n - 1, s_even, b_even, s, base);
            } else {
                s_even = s;
                b_even = base;
            }
        }
        if (N & 1) pair(N - 1, s_even, b_even, f32x4{0.f, 0.f, 0.f, 0.f}, b_even);
    }

    // ---- the split's state -----------------------------------------------------
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 >= rows) return;
    const int rr = row_base + n16;
    const int req = first_req + rr / g;
    const int h = rr % g;
    const int64_t idx = ((int64_t)req * a.part.S + s) * a.Hq + h;
    float *op = a.part.o + idx * DV;
#pragma unroll
    for (int db = 0; db < DB; db++) *(f32x4 *)(op + db * 16 + kq * 4) = oacc[db];
    if (kq == 0) *(float2 *)(a.part.ml + idx * 2) = make_float2(m_run, l);
}

}  // namespace

// Flat (kind 0), prefix (kind 1) and suffix (kind 2) splits over a latent
// cache: Hkv = 1, D = 576 scores / 512 values, Hq a multiple of 16.
int launch_split_mla(const SplitArgs &a0, hipStream_t st) {
    if (a0.n_sets == 0 || a0.max_splits == 0) return SGL_OK;
    if (a0.chunk % MT != 0 || a0.Hq % 16 != 0 || a0.Hkv != 1) return SGL_ERR_INVALID;
    SplitArgs a = a0;
    const int rows = (a.kind == 1 ? a.max_members : 1) * a.Hq;
    a.row_blocks = (rows + 15) / 16;
    const int rbw = a.row_blocks >= 4 ? 4 : (a.row_blocks >= 2 ? 2 : 1);
    const int n_rbg = (a.row_blocks + rbw - 1) / rbw;
    const int64_t n_items = (int64_t)a.n_sets * a.max_splits;   // (set, split) pairs
    const int64_t n_wg = n_items * n_rbg;
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
    if (a.row_blocks >= 4 && a.kind != 1) {
        // 64 or more query rows per split: one wave per 16-row block
        constexpr int FR = 4;
        const int64_t nr = (a.row_blocks + FR - 1) / FR;
        const int64_t n_wf = (nr > 1 ? ceil_div64(n_items, 8) * 8 : n_items) * nr;
        if (n_wf > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
        if (nr > 1) hipLaunchKernelGGL((split_mla_full_kernel<FR, 4, true>), dim3((unsigned)n_wf), dim3(64 * FR), dyn, st, a);
        else hipLaunchKernelGGL((split_mla_full_kernel<FR, 4, false>), dim3((unsigned)n_wf), dim3(64 * FR), dyn, st, a);
        return hip_status(hipGetLastError());
    }
    if (a.kind != 1) {
        // fewer than 64 query rows per split: one wave per 16-row block, one or
        // two blocks per workgroup sharing a two-tile ring
        if (a.row_blocks == 1) {
            hipLaunchKernelGGL((split_mla_full_kernel<1, 2, false>), dim3((unsigned)n_wg), dim3(64), dyn, st, a);
        } else {
            const int64_t nr = (a.row_blocks + 1) / 2;
            const int64_t n_w2 = (nr > 1 ? ceil_div64(n_items, 8) * 8 : n_items) * nr;
            if (n_w2 > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
            if (nr > 1) hipLaunchKernelGGL((split_mla_full_kernel<2, 2, true>), dim3((unsigned)n_w2), dim3(128), dyn, st, a);
            else hipLaunchKernelGGL((split_mla_full_kernel<2, 2, false>), dim3((unsigned)n_w2), dim3(128), dyn, st, a);
        }
        return hip_status(hipGetLastError());
    }
    const dim3 grid((unsigned)n_wg), block(256 * rbw);
    if (rbw == 4) hipLaunchKernelGGL((split_mla_kernel<4>), grid, block, dyn, st, a);
    else if (rbw == 2) hipLaunchKernelGGL((split_mla_kernel<2>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((split_mla_kernel<1>), grid, block, dyn, st, a);
    return hip_status(hipGetLastError());
}
