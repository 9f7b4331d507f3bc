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
// KV head share an XCD and its L2 holds that head's prefix.  Within a
// request the query tiles go last to first (the causal tiles with the most
// keys start first; 1 % shorter on the 64 x 256 over 2048 workload).
//
// Keys are gathered by slot id straight from HBM into LDS with
// global_load_lds_dwordx4 (no register staging), 32 keys at a time, into rings
// of three K tiles and three V tiles.  Such a load writes LDS contiguously by
// lane, so each lane picks WHICH 16-byte chunk of its row it fetches: chunk c
// of row r sits at position c ^ swz(r), an XOR swizzle under which both the
// MFMA operand reads of K and the transposed reads of V are bank-conflict
// free.  The slot ids themselves are copied into a table in LDS (1024 keys,
// refilled half by half for longer contexts), so the loop issues no global
// loads other than the tile loads.
//
// Occupancy is the lever: every wave's per-tile chain (operand reads, eight
// chained MFMAs, the row maximum, the exponentials, eight more MFMAs) is
// latency-bound, and the matrix pipe is kept busy by the other waves of the
// SIMD.  The kernel is sized for three waves per SIMD (three workgroups per
// CU: at most 168 VGPRs and 52 KiB of LDS each), which measured faster than
// two waves per SIMD with a two-stage software pipeline inside each wave.
// Each wave owns 32 query rows; stage n:
//   the first K operand reads of tile n, then the slot-table look-ups and the
//   loads of tile n+2 into the ring slots tile n-1 has left (the two latencies
//   overlap); S^T(n) = K Q^T on MFMA (keys on M, rows on N, so a lane owns one
//   row's scores) with each K read four steps ahead of its MFMA; the causal
//   mask and row maximum; the reference move; p = 2^(s*c - reference), its
//   bf16 copy and its fp32 row sum; O^T += V^T P^T on MFMA (V^T via ds_read_b64_tr_b16, two
//   MFMAs ahead; the key order inside each MFMA matches the S^T accumulator
//   layout, so P needs no lane exchange); the wait for tile n+1; one barrier.
// Every tile load has two stages to land.  Softmax details: Q enters the
// MFMAs exactly as given (a negative scale negates it, which is exact), the
// scores s = q.k come out of the MFMAs in fp32, and the scale joins them in
// fp32 inside the exponent: p = 2^(s*c - reference) with c = |scale|*log2(e),
// one FMA per score.  The reference maximum is moved lazily, only when a
// row's tile maximum exceeds it by more than 2^8 (the exact result is
// unchanged: the reference is only a scaling point): each lane compares the
// maximum of its half of the row's scores, unscaled, with that threshold
// divided by the factor, and only when some lane passes it are the two halves
// combined and scaled; the mask is applied only to tiles that may cross the
// diagonal.  p is rounded to bf16 for the PV MFMAs (the only reduced-
// precision step); the row sum l adds the fp32 p, so the log-sum-exp is that
// of the fp32 scores.
#include <type_traits>

#include "common.h"

namespace {

constexpr int BN = 32;        // keys per LDS tile
constexpr int RING = 3;       // LDS tiles per ring (K and V each)
constexpr int TABH = 512;     // keys per half of the LDS slot-id table
constexpr int BM = kExtendTileRows;   // query rows per workgroup
constexpr int NT = 256;       // threads
constexpr float kLazy = 8.f;  // move the reference only when the max grows by more than 2^8

// Position of 16-byte chunk c of LDS row r is c ^ swz<D>(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void *p) {
    union { uint4 u; bf16x8 b; } x;
    x.u = *(const uint4 *)p;
    return x.b;
}

// Combine lanes l and l^32, which hold the two halves of a row's 32-key block.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int V>
using IC = std::integral_constant<int, V>;

// s_waitcnt vmcnt(N) (lgkmcnt and expcnt left alone), as the builtin so that
// the compiler's own wait insertion knows which loads have completed
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// OFF32: every K/V byte offset fits in 32 bits (num_slots * Hkv * D * 2 <=
// 2^32), so the slot table holds ready byte offsets and a load address is the
// uniform pool base plus a 32-bit per-lane offset.
// SPLIT: the key range of a (request, query tile, KV head) is cut into splits
// of ksplit keys (a multiple of 2 * TABH), one workgroup each, which write
// their partial softmax states (m, l in log2 units, unnormalised o in fp32)
// for the log-sum-exp merge instead of o -- for grids too small to fill the
// chip over long contexts.
template <int D, bool OFF32, bool SPLIT>
__global__ void __launch_bounds__(NT, 3) extend_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k_pool,
    const __bf16 *__restrict__ v_pool, int64_t num_slots, const int32_t *__restrict__ r2t,
    int64_t num_rows, int64_t stride, const int32_t *__restrict__ req_rows,
    const int32_t *__restrict__ prefix_lens, const int64_t *__restrict__ q_off, int Hq, int Hkv,
    int n_qtiles, float qscale, __bf16 *__restrict__ o, float *__restrict__ lse, int batch, int ksplit,
    float *__restrict__ part_o, float *__restrict__ part_ml, int part_S) {
    constexpr int QT = D / 16;            // k-steps of 16 dims for S^T
    constexpr int DBLK = D / 32;          // 32-dim output blocks
    constexpr int ROWB = 2 * D;           // bytes per K or V row of one KV head
    constexpr int CHK = D / 8;            // 16-byte chunks per row
    constexpr int RPB = 64 / CHK;         // rows per 1 KiB direct-load block
    constexpr int NB = BN / RPB / 4;      // 1 KiB blocks per wave per tile (K and V each)
    constexpr int TILEB = BN * ROWB;
    // one LDS object per ring slot, so the compiler can tell that reads of one
    // slot do not wait on the direct loads into another
    __shared__ __attribute__((aligned(16))) unsigned char k_lds0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds1[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds2[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds1[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds2[TILEB];
    auto kbuf = [&](auto i) -> unsigned char * {
        constexpr int I = decltype(i)::value % RING;
        return I == 0 ? k_lds0 : I == 1 ? k_lds1 : k_lds2;
    };
    auto vbuf = [&](auto i) -> unsigned char * {
        constexpr int I = decltype(i)::value % RING;
        return I == 0 ? v_lds0 : I == 1 ? v_lds1 : v_lds2;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int id = blockIdx.x;
    const int kvh = id % Hkv;
    const int rest = id / Hkv;
    const int qt = n_qtiles - 1 - rest % n_qtiles;   // the tiles with the most keys first
    const int r = SPLIT ? (rest / n_qtiles) % batch : rest / n_qtiles;
    const int sp = SPLIT ? rest / n_qtiles / batch : 0;   // split of the key range
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
    // this workgroup's keys [k_lo, k_hi): all of them, or split sp
    const int k_lo = SPLIT ? sp * ksplit : 0;
    if (k_lo >= kv_end) return;
    const int k_hi = SPLIT && k_lo + ksplit < kv_end ? k_lo + ksplit : kv_end;
    const int n0 = k_lo / BN;                        // first key tile (a multiple of 2 TABH / BN)
    const int32_t *row = r2t + rowi * stride;
    const int64_t rowstride_el = (int64_t)Hkv * D;

    // ---- this lane's query row ------------------------------------------------
    const int n32 = lane & 31, h2 = lane >> 5;
    const int rho = wave * 32 + n32;                 // row in the tile
    const int tok_local = q0 + rho / g;              // new-token index within the request
    const bool row_valid = tok_local < E;
    const int h = kvh * g + rho % g;
    const int pos = P + (row_valid ? tok_local : E - 1);   // absolute position
    // q as given; negated (exactly) when the scale is negative, so that the
    // scaled score is |scale| * (q.k) with a positive factor
    bf16x8 qf[QT];
    {
        const __bf16 *src = q + ((t0 + (row_valid ? tok_local : 0)) * Hq + h) * D + 8 * h2;
        const bool neg = qscale < 0.f;
#pragma unroll
        for (int t = 0; t < QT; t++) {
            qf[t] = ld_bf16x8(src + 16 * t);
            if (neg) qf[t] = -qf[t];
        }
    }
    const float cs = fabsf(qscale);   // |scale| * log2(e): scores -> log2 units
    const float inv_cs = 1.f / cs;

    f32x16 oacc[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; b++)
#pragma unroll
        for (int j = 0; j < 16; j++) oacc[b][j] = 0.f;
    float m_run = -INFINITY;     // reference maximum (log2 units of the scaled score)
    float m_sub = 0.f;           // the reference as subtracted before 2^x (0 while none)
    float l_run = 0.f;           // this lane's part of the row sum
    float thr = -INFINITY;       // a tile maximum above this moves the reference
    float thr_s = -INFINITY;     // the same threshold in raw score units (thr / cs)

    // ---- slot ids: a table in LDS holds the ids of keys [c*TABH, (c+1)*TABH)
    // in half c % 2, so the loop reads them from LDS instead of HBM.  The
    // first two chunks are filled here; a longer context refills a half once
    // its last key has been looked up (every TABH / BN stages).
    // Entries past the end hold the last key's slot, so look-ups need no
    // clamp (a tile past the end is a harmless copy of that key).  With 32-bit
    // offsets the table stores the byte offset of the slot's row of this KV
    // head (an id outside the pool is replaced by slot 0).
    using TabT = typename std::conditional<OFF32, uint32_t, int32_t>::type;
    __shared__ TabT slot_tab[2 * TABH];
    const char *row_b = (const char *)row;
    const uint32_t rowbytes = (uint32_t)rowstride_el * 2u;
    const uint32_t ns32 = OFF32 ? (uint32_t)num_slots : 0u;
    auto fill = [&](auto count_tag, int k0) {        // keys k0 .. k0 + count*NT - 1
        constexpr int CNT = decltype(count_tag)::value;
        int v[CNT];
#pragma unroll
        for (int u = 0; u < CNT; u++) {
            const int k = min(k0 + u * NT + tid, k_hi - 1);
            v[u] = *(const int32_t *)(row_b + (uint32_t)k * 4u);
        }
#pragma unroll
        for (int u = 0; u < CNT; u++) {
            TabT e;
            if (OFF32) e = ((uint32_t)v[u] < ns32 ? (uint32_t)v[u] : 0u) * rowbytes + (uint32_t)(kvh * D * 2);
            else e = v[u];
            slot_tab[(k0 + u * NT + tid) & (2 * TABH - 1)] = e;
        }
    };

    // ---- tile loader: wave w fills 1 KiB blocks w*NB .. w*NB+NB-1 of a tile ---
    // lane -> (row rr = block * RPB + lane / CHK, position lane % CHK),
    // fetching chunk (lane % CHK) ^ swz(rr) of key tile*BN + rr (clamped to
    // the last key, so tiles past the end are harmless copies).
    int jl[NB];                  // this lane's key within a tile, per block
    uint32_t lp[NB];             // byte offset of this lane's chunk within a K/V row
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int rr = (wave * NB + i) * RPB + lane / CHK;
        jl[i] = rr;
        lp[i] = (uint32_t)(8 * ((lane % CHK) ^ swz<D>(rr))) * 2u;
    }
    using Off = typename std::conditional<OFF32, uint32_t, int64_t>::type;
    // pool byte offsets of this lane's rows of tile `tile` (a K tile and the V
    // tile of the same keys share them)
    auto offsets = [&](int tile, Off (&dst)[NB]) {
        // tile * BN is a multiple of BN and jl[i] < BN, so the wrap of the
        // table index touches only the uniform part
        const TabT *tab = slot_tab + ((tile * BN) & (2 * TABH - 1));
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const TabT e = tab[jl[i]];
            if (OFF32) dst[i] = e + lp[i];
            else dst[i] = (int64_t)safe_slot(e, num_slots) * rowstride_el * 2 + (kvh * D * 2 + lp[i]);
        }
    };
    auto issue = [&](const __bf16 *pool, unsigned char *dst, const Off (&off)[NB]) {
#pragma unroll
        for (int i = 0; i < NB; i++)
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)((const char *)pool + off[i]),
                                             (SGL_LDS void *)(dst + (wave * NB + i) * 1024), 16, 0, 0);
    };

    // Per-lane LDS byte offsets of the MFMA operand reads.  The swizzle of a
    // row depends only on bits that stay fixed across the 16-row V steps, so
    // the step index becomes an immediate offset.
    const int grp = (lane >> 4) & 1;                 // which 16 dims of a 32-dim block
    const int r4 = (lane & 15) >> 2, qq = lane & 3;
    int koff[QT];                                    // K operand of step t
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

    // S^T of one tile (K operands from LDS, Q from registers)
    // (the first KA operand reads go out before the slot-table look-ups and
    // the tile loads, held there by a fence; inside the MFMA loop the compiler
    // places the remaining reads, which measured ~1 % faster than fencing
    // every step)
    constexpr int KA = 4;
    auto k_first = [&](const unsigned char *kt, bf16x8 (&ka)[KA]) {
#pragma unroll
        for (int t = 0; t < KA; t++) ka[t] = ld_bf16x8(kt + koff[t]);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto s_tile = [&](const unsigned char *kt, bf16x8 (&ka)[KA]) {
        f32x16 s = {};
#pragma unroll
        for (int t = 0; t < QT; t++) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % KA], qf[t], s, 0, 0, 0);
            if (t + KA < QT) ka[t % KA] = ld_bf16x8(kt + koff[t + KA]);
        }
        return s;
    };
    // causal mask of tile n (absolute key of accumulator element j:
    // 32n + 8*(j/4) + 4*h2 + j%4) and the maximum of this lane's 16 scores
    auto mask_max = [&](f32x16 &s, int n, auto mask_tag) {
        if (decltype(mask_tag)::value) {
            const int lim = pos - n * BN - 4 * h2;
#pragma unroll
            for (int j = 0; j < 16; j++)
                if (8 * (j >> 2) + (j & 3) > lim) s[j] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int j = 1; j < 16; j++) mx = fmaxf(mx, s[j]);
        return mx;               // this lane's half of the row, raw score units
    };
    // lazy move of the reference (mx_half: this lane's half-row maximum of
    // the tile); rescales O and l, so it runs after the PV MFMAs issued before it
    auto move_ref = [&](float mx_half) {
        if (__builtin_amdgcn_ballot_w64(mx_half > thr_s)) {
            const float mx = max_xor32(mx_half) * cs;   // the whole row's maximum, log2 units
            const bool need = mx > thr;
            const float m_new = need ? mx : m_run;
            const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < DBLK; b++) oacc[b] *= alpha;
            m_run = m_new;
            m_sub = m_new == -INFINITY ? 0.f : m_new;
            thr = m_new + kLazy;
            thr_s = thr * inv_cs;
        }
    };
    // p = 2^(s*cs - reference) in fp32, rounded to bf16 for the B operands of
    // the tile's 2 PV steps; the row sum adds the fp32 values (a pairwise tree,
    // so the additions do not form one long dependent chain)
    auto exp_tile = [&](const f32x16 &s, bf16x8 (&pf)[2]) {
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            p[j] = __builtin_amdgcn_exp2f(fmaf(s[j], cs, -m_sub));
            pf[j >> 3][j & 7] = (__bf16)p[j];
        }
#pragma unroll
        for (int w = 1; w < 16; w *= 2)
#pragma unroll
            for (int j = 0; j < 16; j += 2 * w) p[j] += p[j + w];
        l_run += p[0];
    };
    // O^T += V^T P^T; step s2 covers keys 16*s2 + {4*h2 + 0..3, 8 + 4*h2 + 0..3}
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    constexpr int VA = 2;
    // operand of PV MFMA i = s2 * DBLK + b.  TAIL: a tile that may end before
    // BN keys (nv valid): the values of the missing keys are replaced by zeros
    // in registers (their p is 0, and the rows they were loaded from must not
    // turn 0 * v into NaN)
    auto v_op = [&](const unsigned char *vt, int i, int nv, auto tail_tag) {
        const int s2 = i / DBLK, b = i % DBLK;
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)(vt + s2 * 16 * ROWB + voff0[b]));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)(vt + s2 * 16 * ROWB + voff1[b]));
        i16x8 cat = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        if (decltype(tail_tag)::value) {
#pragma unroll
            for (int e = 0; e < 8; e++)         // element e holds key 16 s2 + 8 (e / 4) + 4 h2 + e % 4
                if (16 * s2 + 8 * (e >> 2) + 4 * h2 + (e & 3) >= nv) cat[e] = 0;
        }
        return __builtin_bit_cast(bf16x8, cat);
    };
    auto pv_tile = [&](const unsigned char *vt, const bf16x8 (&pf)[2], int nv, auto tail_tag) {
        bf16x8 va[VA];
#pragma unroll
        for (int i = 0; i < VA; i++) va[i] = v_op(vt, i, nv, tail_tag);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * DBLK; i++) {
            oacc[i % DBLK] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % VA], pf[i / DBLK], oacc[i % DBLK], 0, 0, 0);
            if (i + VA < 2 * DBLK) va[i % VA] = v_op(vt, i + VA, nv, tail_tag);
        }
    };

    const int N = (k_hi + BN - 1) / BN;              // key tiles end (tiles n0 .. N-1)
    const int min_pos = P + q0;                      // smallest position in the tile
    // Workgroup barrier for LDS reuse.  __syncthreads (or any LDS release
    // fence) would also wait for every direct load still meant to be in
    // flight, since those write LDS; here the LDS reads are drained and the
    // direct loads are waited for by count (vm_wait) before each barrier.
    auto lds_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- prologue: slot table, then tiles n0 and n0 + 1 (K and V)
    fill(IC<2 * TABH / NT>{}, k_lo);
    __syncthreads();
    Off off[NB];
    offsets(n0, off);
    issue(k_pool, k_lds0, off);
    issue(v_pool, v_lds0, off);
    offsets(n0 + 1, off);
    issue(k_pool, k_lds1, off);
    issue(v_pool, v_lds1, off);
    vm_wait<2 * NB>();           // tile n0
    lds_barrier();

    // ---- stage n (R = (n - n0) % RING): the loads of tile n+2 into the ring
    // slots tile n-1 has left; S^T of tile n, its mask and row maximum, the
    // reference move, p, and PV; then the wait for tile n+1 and one barrier.
    // One chain per wave: the other waves on the SIMD (three per SIMD) fill
    // the matrix pipe meanwhile.  MASK: tile n may cross the diagonal.
    auto stage = [&](const int n, auto r_tag, auto mask_tag) {
        constexpr int R = decltype(r_tag)::value;
        // the first K operand reads go out before the slot-table look-ups of
        // the loads, so the two latencies overlap
        bf16x8 ka[KA];
        k_first(kbuf(IC<R>{}), ka);
        offsets(n + 2, off);
        issue(k_pool, kbuf(IC<R + 2>{}), off);
        issue(v_pool, vbuf(IC<R + 2>{}), off);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s = s_tile(kbuf(IC<R>{}), ka);
        move_ref(mask_max(s, n, mask_tag));
        bf16x8 pf[2];
        exp_tile(s, pf);
        pv_tile(vbuf(IC<R>{}), pf, k_hi - n * BN, mask_tag);
        vm_wait<2 * NB>();       // tile n+1 has landed
        lds_barrier();
    };
    // the slot table's half that held chunk c - 2 takes chunk c once the
    // last look-up of chunk c - 2 (tile SPC c - SPC - 1, at stage SPC c - SPC - 3)
    // is done; chunk c's first look-up comes SPC - 1 stages later
    constexpr int SPC = TABH / BN;                   // tiles per chunk
    int fill_c = k_lo / TABH + 2;
    auto refill = [&](int n_next) {
        if (n_next >= SPC * (fill_c - 1) - 2 && fill_c * TABH < k_hi) {
            fill(IC<TABH / NT>{}, fill_c * TABH);
            ++fill_c;
        }
    };
    // tiles wholly at or below every row's position need no mask; the loops
    // run in groups of RING so that ring positions are known at compile time
    const int n_free = min_pos >= 31 ? (min_pos - 31) / BN + 1 : 0;   // tiles 0 .. n_free-1 need no mask
    const int n_unmasked = n0 + min(max(n_free - n0, 0) / RING * RING, (N - n0) / RING * RING);
    int n = n0;
    for (; n < n_unmasked; n += RING) {
        stage(n, IC<0>{}, std::false_type{});
        stage(n + 1, IC<1>{}, std::false_type{});
        stage(n + 2, IC<2>{}, std::false_type{});
        refill(n + RING);
    }
    for (; n < N; n += RING) {
        stage(n, IC<0>{}, std::true_type{});
        if (n + 1 < N) stage(n + 1, IC<1>{}, std::true_type{});
        if (n + 2 < N) stage(n + 2, IC<2>{}, std::true_type{});
        refill(n + RING);
    }
    vm_wait<0>();                // the trailing clamped loads

    // ---- epilogue: normalise and store ----------------------------------------
    const float l = add_xor32(l_run);
    if (!row_valid) return;
    if constexpr (SPLIT) {
        const int64_t idx = ((t0 + tok_local) * part_S + sp) * Hq + h;
        float *op = part_o + idx * D;
#pragma unroll
        for (int b = 0; b < DBLK; b++)
#pragma unroll
            for (int a4 = 0; a4 < 4; a4++)
                *(f32x4 *)(op + b * 32 + 8 * a4 + 4 * h2) =
                    f32x4{oacc[b][a4 * 4], oacc[b][a4 * 4 + 1], oacc[b][a4 * 4 + 2], oacc[b][a4 * 4 + 3]};
        if (h2 == 0) *(float2 *)(part_ml + idx * 2) = make_float2(m_run, l);
        return;
    }
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
                       float scale, __bf16 *o, float *lse, int32_t n_split, int32_t ksplit, PartialBuf part,
                       hipStream_t st) {
    if (batch == 0 || max_extend_len == 0) return SGL_OK;
    if (row_stride > 0x7fffffff) return SGL_ERR_UNSUPPORTED;   // positions are 32-bit in the kernel
    if (n_split > 1 && (ksplit <= 0 || ksplit % (2 * TABH) != 0 || !part.o || !part.ml || part.S < n_split))
        return SGL_ERR_INVALID;
    const int g = Hq / Hkv;
    const int tok_per_tile = BM / g;
    const int n_qtiles = (int)ceil_div64(max_extend_len, tok_per_tile);
    const int64_t n_wg = (int64_t)n_qtiles * batch * Hkv * (n_split > 1 ? n_split : 1);
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const float qs = scale * kLog2e;
    const bool off32 = num_slots * Hkv * D * 2 <= (int64_t(1) << 32);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(NT), 0, st, q, k_pool, v_pool, num_slots, r2t,
                           num_rows, row_stride, req_rows, prefix_lens, q_off, Hq, Hkv, n_qtiles, qs, o, lse, batch,
                           ksplit, part.o, part.ml, (int)part.S);
    };
    const bool split = n_split > 1;
    if (D == 128) {
        if (off32) split ? go(extend_bf16_kernel<128, true, true>) : go(extend_bf16_kernel<128, true, false>);
        else split ? go(extend_bf16_kernel<128, false, true>) : go(extend_bf16_kernel<128, false, false>);
    } else {
        if (off32) split ? go(extend_bf16_kernel<64, true, true>) : go(extend_bf16_kernel<64, true, false>);
        else split ? go(extend_bf16_kernel<64, false, true>) : go(extend_bf16_kernel<64, false, false>);
    }
    return hip_status(hipGetLastError());
}
