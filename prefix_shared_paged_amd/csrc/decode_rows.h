// decode_rows.h -- work item of the whole-row split-K decode (kernels_decode_rows.hip),
// as a device function so that a kernel can run it beside other stages.
//
// A pool row holds all KV heads of one slot (layout [num_slots, Hkv, D]):
// 2 KiB for Hkv = 8, D = 128 in bf16, 1 KiB in fp8.  On MI355X random gathers
// of whole rows reach about 6.8 TB/s, while gathers of one head's 128 or 256
// bytes per row reach about 5.5 and 6.4 TB/s.  Decode is a pure gather of
// such rows ("SGLang 深度拆解" section 4.1: decode reads the whole KV and is
// memory-bound), so here the HPW waves of a workgroup -- wave w owns KV head
// hg * HPW + w and its Hq/Hkv query rows -- load rows together: every
// direct-to-LDS instruction moves 1 KiB of consecutive tile rows
// (non-temporal), the waves share the tile, and each wave reads its own
// head's part of it.  Per tile the arithmetic is that of the per-head kernels
// in kernels_decode.hip (bf16: 16-key tiles; fp8: 32-key tiles widened to
// bf16 in registers); the workgroup meets at a barrier before a tile buffer
// is read and before it is refilled.
#pragma once

#include "common.h"
#include "decode_util.h"

namespace sgl_decode {

// Position of 16-byte chunk c (counted over the whole row) of tile row r is
// c ^ rsw(r), masked to the row's CR chunks.  Rows are at least 256 bytes
// apart, so a chunk's LDS bank group (of 16) is its position's low four bits:
// the four-bit swizzle spreads the 16 rows of a K operand read and the rows
// of a transposed V read over distinct bank groups.
constexpr int kRowsHeads = 4;   // KV heads per workgroup (at most)

template <bool FP8, int CR>
__device__ __forceinline__ int rsw(int r) {
    const int f = FP8 ? ((r & 15) ^ ((r >> 4) << 2)) : (((r & 7) << 1) | ((r >> 3) & 1));
    return f & (CR - 1);
}

// Work item of id bid: split round s and work set v (below).
__device__ __forceinline__ void rows_item(const SplitArgs &a, int HPW, int bid, int &s, int &v) {
    const int n_v = a.n_sets * (a.Hkv / HPW);
    const int rb = a.xcd_block;
    const int bpx = ((n_v + rb - 1) / rb + 7) / 8;        // blocks per XCD and round
    const int xcd = (int)((unsigned)bid & 7u);
    const int local = (int)((unsigned)bid >> 3);
    s = local / (bpx * rb);
    const int sl = local % (bpx * rb);
    const int b = (sl / rb) * 8 + ((xcd - s) & 7);
    v = b * rb + sl % rb;
}

// Whether item bid of a suffix stage (kind 2 with suffix starts) has keys:
// the test rows_split makes before its work, for one item per lane.
__device__ __forceinline__ bool rows_item_live(const SplitArgs &a, int HPW, int bid) {
    int s, v;
    rows_item(a, HPW, bid, s, v);
    if (s >= a.max_splits || s >= a.part.S || v >= a.n_sets * (a.Hkv / HPW)) return false;
    const int set = v % a.n_sets;
    const int64_t L = a.seq_lens[set], P = a.suffix_lo[set], row = a.req_rows[set];
    if (row < 0 || row >= a.num_rows) return false;
    const int64_t lo = P < 0 ? 0 : (P > L ? L : P), hi = L < a.row_stride ? L : a.row_stride;
    return s < ceil_div64(hi - lo, a.chunk);
}

template <int D, bool FP8, int HPW, bool LONG = false>
__device__ __forceinline__ void rows_segment(const SplitArgs &a, int tid, int set, int hg, int64_t ref_row,
                                             int64_t k0, int nk, int64_t part_row, unsigned char *k_lds,
                                             unsigned char *v_lds, int32_t *slot_lds);

// HPW waves per workgroup, one per KV head of the head group hg: the
// workgroup loads the group's HPW * D * elt bytes of every row (the whole row
// when HPW = Hkv).
//
// bid is the work item's id (the workgroup id, less the workgroups of other
// stages that precede it in a shared grid, which come in multiples of 8, so
// bid % 8 is still the XCD); tid is threadIdx.x (a caller that runs several
// items in a loop passes a copy the compiler cannot see through, so that
// nothing derived from it is kept live across the loop); k_lds and v_lds
// hold one tile each (T * R bytes), slot_lds a.chunk slot ids.
template <int D, bool FP8, int HPW>
__device__ __forceinline__ void rows_split(const SplitArgs &a, int bid, int tid, unsigned char *k_lds,
                                           unsigned char *v_lds, int32_t *slot_lds) {
    // ---- work item (uniform over the workgroup): split s of (request, head group)
    // The work sets are v = hg * n_sets + request; they form blocks of rb
    // consecutive ones (one head group of rb consecutive requests).
    // Workgroups go to the 8 XCDs round-robin by id (id % 8 is the XCD), and
    // each XCD runs its workgroups in id order.  Split round s gives block b
    // to XCD (b + s) % 8: the rotation spreads every set's splits over the
    // XCDs (an XCD's total work does not hang on the lengths of a few
    // requests), and with rb > 1 sibling requests (adjacent in the batch)
    // still read the prefix rows of one split through one XCD's L2.  Rounds
    // are in order, so every set's first split starts before any second one.
    const int ng = a.Hkv / HPW;
    const int n_v = a.n_sets * ng;
    int s, v;
    rows_item(a, HPW, bid, s, v);
    if (s >= a.max_splits || v >= n_v) return;
    const int set = v % a.n_sets, hg = v / a.n_sets;
    const int64_t L = a.seq_lens[set];
    const int64_t ref_row = a.req_rows[set];
    int64_t lo = 0, hi = L;
    if (a.kind == 2) {
        const int64_t P = a.suffix_lo ? a.suffix_lo[set] : a.group_prefix_len[wave_find_group(a.group_ptr, a.G, set)];
        lo = P < 0 ? 0 : (P > L ? L : P);
    }
    if (ref_row < 0 || ref_row >= a.num_rows) return;
    if (hi > a.row_stride) hi = a.row_stride;
    const int64_t n_split = ceil_div64(hi - lo, a.chunk);
    if (s >= n_split || s >= a.part.S) return;
    const int64_t k0 = lo + (int64_t)s * a.chunk;
    const int nk = (int)((k0 + a.chunk < hi ? k0 + a.chunk : hi) - k0);
    rows_segment<D, FP8, HPW>(a, tid, set, hg, ref_row, k0, nk, (int64_t)set * a.part.S + s, k_lds, v_lds,
                              slot_lds);
}

// Keys [k0, k0 + nk) of request `set`'s row ref_row for the KV heads of head
// group hg: the tile loop of one work item, writing the partial state of
// every query row to state row `part_row` of a.part (index part_row * Hq +
// query head).  Uniform over the workgroup.  The slot table holds a.chunk
// ids (a multiple of the tile): nk <= a.chunk, or, with LONG, any nk, the
// table then being refilled every a.chunk keys.
template <int D, bool FP8, int HPW, bool LONG>
__device__ __forceinline__ void rows_segment(const SplitArgs &a, int tid, int set, int hg, int64_t ref_row,
                                             int64_t k0, int nk, int64_t part_row, unsigned char *k_lds,
                                             unsigned char *v_lds, int32_t *slot_lds) {
    constexpr int ELT = FP8 ? 1 : 2;
    constexpr int T = FP8 ? 32 : 16;        // keys per tile
    constexpr int R = HPW * D * ELT;        // bytes of one tile row (the group's heads of a slot)
    constexpr int CR = R / 16;              // 16-byte chunks per tile row
    constexpr int HC = D * ELT / 16;        // chunks per head
    constexpr int TB = T * R;               // bytes of one K (or V) tile
    constexpr int NI = TB / 1024;           // 1 KiB direct-load instructions per tile
    static_assert(TB % 1024 == 0 && NI % HPW == 0, "whole load instructions per wave");
    constexpr int NIW = NI / HPW;
    constexpr int QT = D / 32;              // MFMA k-steps over head_dim
    constexpr int DB = D / 16;              // 16-dim output blocks
    constexpr int KCH = D / 64;             // fp8: K chunks per lane per 16-key block

    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // head of this wave in its group
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    const int kvh = hg * HPW + w;                   // KV head of this wave
    const int N = (nk + T - 1) / T;                 // tiles, >= 1
    const int g = a.Hq / a.Hkv;                     // query rows of this wave (<= 16)

    const int32_t *row = a.r2t + ref_row * a.row_stride + k0;
    // LONG: the table holds keys [sub, sub + a.chunk) of the segment
    int sub = 0;
    auto fill = [&](int base) {
        const int cnt = LONG ? min(nk - base, a.chunk) : nk;
        for (int j = tid; j < cnt; j += 64 * HPW) slot_lds[j] = safe_slot(row[base + j], a.num_slots);
    };
    fill(0);

    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand of query row n16 (head kvh*g + n16) -------------------------
    // bf16: step t holds dims 32t + 8kq + i;  fp8: dims kq*D/4 + 8t + i
    bf16x8 qf[QT];
    {
        const int h = kvh * g + (n16 < g ? n16 : 0);
        const __bf16 *src = (const __bf16 *)a.q + ((int64_t)set * a.Hq + h) * D;
#pragma unroll
        for (int t = 0; t < QT; t++) qf[t] = ld_q(src + (FP8 ? kq * (D / 4) + 8 * t : 32 * t + 8 * kq));
        if (n16 >= g)
#pragma unroll
            for (int t = 0; t < QT; t++) qf[t] = bf16x8{};
    }

    // ---- direct loads: instruction ii = u*HPW + w of a tile covers its bytes
    // [1024 ii, 1024 ii + 1024); lane -> tile row, LDS chunk position, and the
    // chunk of the group's part of the pool row that belongs there
    int lrow[NIW], lsrc[NIW];
#pragma unroll
    for (int u = 0; u < NIW; u++) {
        const int off = (u * HPW + w) * 1024 + 16 * lane;
        lrow[u] = off / R;
        lsrc[u] = 16 * (((off % R) / 16) ^ rsw<FP8, CR>(lrow[u]));
    }
    const int64_t pool_row = (int64_t)a.Hkv * D * ELT;   // bytes per slot
    const char *kp = (const char *)a.k_pool + hg * R;
    const char *vp = (const char *)a.v_pool + hg * R;

    __syncthreads();   // slot table visible

    auto issue = [&](int n, const char *pool, unsigned char *dst) {
#pragma unroll
        for (int u = 0; u < NIW; u++) {
            const int kk = min(n * T + lrow[u], nk - 1);   // past the split end: repeat the last key
            const char *src = pool + (int64_t)slot_lds[LONG ? kk - sub : kk] * pool_row + lsrc[u];
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                             (SGL_LDS void *)(dst + (u * HPW + w) * 1024), 16, 0, 2 /* nt */);
        }
    };
    // LDS byte address of chunk c of this wave's head in tile row r
    auto at = [&](uint32_t base, int r, int c) { return base + r * R + 16 * ((w * HC + c) ^ rsw<FP8, CR>(r)); };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float qscale = FP8 ? a.scale * kLog2e * a.k_scale[kvh] : a.scale * kLog2e;

    constexpr int NB = FP8 ? 2 : 1;   // 16-key S blocks per tile
    // S^T = K Q^T: block b, lane (row n16, kq) gets 4 keys (see key_of)
    auto s_tile = [&](f32x4 (&sacc)[NB]) {
        const uint32_t kb = lds_addr(k_lds);
        if constexpr (FP8) {
            uint32_t ad[2 * KCH];
#pragma unroll
            for (int b = 0; b < 2; b++)
#pragma unroll
                for (int c = 0; c < KCH; c++)
                    ad[b * KCH + c] = at(kb, 8 * (n16 >> 2) + 4 * b + (n16 & 3), KCH * kq + c);
            u32x4 raw[2 * KCH];
            lds_read_raw128(raw, ad);
#pragma unroll
            for (int b = 0; b < 2; b++) {
                sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < QT; t++) {
                    const u32x4 &r = raw[b * KCH + (t >> 1)];
                    const bf16x8 kf = (t & 1) ? fp8x8_to_bf16(r[2], r[3]) : fp8x8_to_bf16(r[0], r[1]);
                    sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t], sacc[b], 0, 0, 0);
                }
            }
        } else {
            uint32_t ad[QT];
#pragma unroll
            for (int t = 0; t < QT; t++) ad[t] = at(kb, n16, 4 * t + kq);
            bf16x8 kf[QT];
            lds_read_b128(kf, ad);
            sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < QT; t++)
                sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t], qf[t], sacc[0], 0, 0, 0);
        }
    };
    // tile key of accumulator entry j of block b for this lane
    auto key_of = [&](int b, int j) { return FP8 ? 8 * kq + 4 * b + j : 4 * kq + j; };
    // online softmax of the row over tile n (lazy reference maximum, as in
    // kernels_decode.hip), then O^T += V^T P^T
    auto pv_tile = [&](int n, const f32x4 (&sacc)[NB]) {
        float sv[4 * NB];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = n * T + key_of(b, j) < nk ? sacc[b][j] * qscale : -INFINITY;
                sv[4 * b + j] = x;
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
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
            m_run = m_new;
        }
        const uint32_t vb = lds_addr(v_lds);
        if constexpr (FP8) {
            bf16x8 pf;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float pj = __builtin_amdgcn_exp2f(sv[j] - m_run);
                l_run += pj;
                pf[j] = (__bf16)pj;
            }
            // lane (n16, kq) addresses row 8kq + n16/2, half n16%2 of chunk db;
            // the transposed result is dim 16db + n16, keys 8kq .. 8kq + 7
            uint32_t ad[DB];
#pragma unroll
            for (int db = 0; db < DB; db++) ad[db] = at(vb, 8 * kq + (n16 >> 1), db) + 8 * (n16 & 1);
            i32x2 vt[DB];
            lds_read_tr8(vt, ad);
#pragma unroll
            for (int db = 0; db < DB; db++)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(vt[db][0], vt[db][1]), pf,
                                                                    oacc[db], 0, 0, 0);
        } else {
            bf16x4 pf;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float pj = __builtin_amdgcn_exp2f(sv[j] - m_run);
                l_run += pj;
                pf[j] = (__bf16)pj;
            }
            // lane (r4, qq) of group kq reads 4 dims of row 4kq + r4; the
            // transposed result is dim 16db + n16, keys 4kq .. 4kq + 3
            const int r4 = n16 >> 2, qq = n16 & 3;
            uint32_t ad[DB];
#pragma unroll
            for (int db = 0; db < DB; db++) ad[db] = at(vb, 4 * kq + r4, 2 * db + (qq >> 1)) + 8 * (qq & 1);
            i16x4 vt[DB];
            lds_read_tr16(vt, ad);
#pragma unroll
            for (int db = 0; db < DB; db++)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[db], __builtin_bit_cast(i16x4, pf),
                                                                     oacc[db], 0, 0, 0);
        }
    };

    issue(0, kp, k_lds);
    issue(0, vp, v_lds);
    for (int n = 0; n < N; n++) {
        vm_wait<0>();                                // this wave's loads of tile n have landed
        barrier();                                   // ... and every wave's
        f32x4 sacc[NB];
        s_tile(sacc);
        if (n + 1 < N) {
            barrier();                               // every wave has read the K tile
            if (LONG && (n + 1) * T - sub == a.chunk) {
                // tile n + 1 starts the next a.chunk keys: every wave is done
                // with this table (tile n's loads went out in the last pass)
                sub += a.chunk;
                fill(sub);
                __syncthreads();
            }
            issue(n + 1, kp, k_lds);
        }
        pv_tile(n, sacc);
        if (n + 1 < N) {
            barrier();                               // every wave has read the V tile
            issue(n + 1, vp, v_lds);
        }
    }

    // ---- the split's state (m, l, o) of each query row --------------------------
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 >= g) return;
    const float vscale = FP8 ? a.v_scale[kvh] : 1.f;
    const int h = kvh * g + n16;
    const int64_t idx = part_row * a.Hq + h;
    float *op = a.part.o + idx * D;
#pragma unroll
    for (int db = 0; db < DB; db++) *(f32x4 *)(op + db * 16 + kq * 4) = FP8 ? oacc[db] * vscale : oacc[db];
    if (kq == 0) *(float2 *)(a.part.ml + idx * 2) = make_float2(m_run, l);
}

// Run w of the balanced suffix stage for head group hg (see
// kernels_decode_rows.hip): the keys [w C, (w + 1) C) of the concatenated
// suffixes (plan = a.sk_plan), piece by piece, each piece's states in row
// request + w of a.part.  Uniform over the workgroup; each piece takes the
// thread id and the arguments through values the compiler cannot see
// through, so that nothing derived from them stays live across the loop.
typedef const __attribute__((address_space(4))) SplitArgs *KArgs;   // arguments in the kernarg segment
template <int D, bool FP8, int HPW>
__device__ __forceinline__ void balanced_run(KArgs ap, int64_t w, int hg, unsigned char *k_lds,
                                             unsigned char *v_lds, int32_t *slot_lds) {
    const SplitArgs &a = *(const SplitArgs *)ap;
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
        KArgs kp = ap;
        asm volatile("" : "+v"(tid), "+s"(kp));
        rows_segment<D, FP8, HPW, true>(*(const SplitArgs *)kp, tid, r, hg, a.req_rows[r], lo + (p - r_off),
                                        (int)(pe - p), r + w, k_lds, v_lds, slot_lds);
        p = pe;
        if (p >= end) break;
        while (plan[r + 1] <= p) r++;              // the next request with keys (plan[batch] > p)
        __syncthreads();                            // tiles and slot table free for the next piece
    }
}

}  // namespace sgl_decode
