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
// Keys are gathered by slot id straight from HBM into LDS with
// global_load_lds_dwordx4 (no register staging), 32 keys at a time, into rings
// of four K tiles and four V tiles.  Such a load writes LDS contiguously by
// lane, so each lane picks WHICH 16-byte chunk of its row it fetches: chunk c
// of row r sits at position c ^ swz(r), an XOR swizzle under which both the
// MFMA operand reads of K and the transposed reads of V are bank-conflict
// free.  The slot ids themselves are copied once into a table in LDS (4096
// keys, refilled half by half for longer contexts), so the loop issues no
// global loads other than the tile loads.
//
// Each wave owns 32 query rows and walks the keys one 32-key tile at a time
// with a two-stage software pipeline, so that the matrix pipe always has
// independent work while the vector ALU runs the softmax:
//   stage n, part 1: S^T(n+1) = K Q^T on MFMA (keys on M, rows on N, so a lane
//                    owns one row's scores)  ||  p = 2^s of tile n, its bf16
//                    rounding and row sum;
//   stage n, part 2: O^T += V^T P^T of tile n on MFMA (V^T via
//                    ds_read_b64_tr_b16; the key order inside each MFMA matches
//                    the S^T accumulator layout, so P needs no lane exchange)
//                    ||  tile n+1's causal mask and row maximum;
//   then the loads of K tile n+4 and V tile n+3 into the ring slots that K
//   tile n and V tile n-1 have left, and one barrier.
// Every tile load thus has two stages to land.  Softmax details: Q is
// pre-multiplied by scale*log2(e), so scores come out in log2 units; the
// running reference maximum enters as the accumulator input of the first
// S^T MFMA, so p = 2^s needs no further arithmetic; the reference is moved
// lazily, only when a row's tile maximum exceeds it by more than 2^8 (the
// exact result is unchanged: the reference is only a scaling point), and the
// mask is applied only to tiles that may cross the diagonal.
#include <type_traits>

#include "common.h"

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int BN = 32;        // keys per LDS tile
constexpr int RING = 4;       // LDS tiles per ring (K and V each)
constexpr int TABH = 2048;    // keys per half of the LDS slot-id table
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
__global__ void __launch_bounds__(NT, 2) extend_bf16_kernel(
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
    __shared__ __attribute__((aligned(16))) unsigned char k_lds3[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds1[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds2[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds3[TILEB];
    auto kbuf = [&](auto i) -> unsigned char * {
        constexpr int I = decltype(i)::value % RING;
        return I == 0 ? k_lds0 : I == 1 ? k_lds1 : I == 2 ? k_lds2 : k_lds3;
    };
    auto vbuf = [&](auto i) -> unsigned char * {
        constexpr int I = decltype(i)::value % RING;
        return I == 0 ? v_lds0 : I == 1 ? v_lds1 : I == 2 ? v_lds2 : v_lds3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int id = blockIdx.x;
    const int kvh = id % Hkv;
    const int rest = id / Hkv;
    const int qt = rest % n_qtiles;
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
    bf16x8 qf[QT];
    {
        const __bf16 *src = q + ((t0 + (row_valid ? tok_local : 0)) * Hq + h) * D + 8 * h2;
#pragma unroll
        for (int t = 0; t < QT; t++) {
            const bf16x8 raw = ld_bf16x8(src + 16 * t);
#pragma unroll
            for (int e = 0; e < 8; e++) qf[t][e] = (__bf16)((float)raw[e] * qscale);
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; b++)
#pragma unroll
        for (int j = 0; j < 16; j++) oacc[b][j] = 0.f;
    float m_run = -INFINITY;     // reference maximum (log2 units of the scaled score)
    float l_run = 0.f;           // this lane's part of the row sum
    // -reference, broadcast: the accumulator input of the first S^T MFMA, so
    // scores come out relative to the reference (0 until the first tile,
    // which always moves it)
    f32x16 mneg;
#pragma unroll
    for (int j = 0; j < 16; j++) mneg[j] = 0.f;
    float thr = -INFINITY;       // a tile maximum above this moves the reference

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
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const TabT e = slot_tab[(tile * BN + jl[i]) & (2 * TABH - 1)];
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
    // V rows past the end of the context must hold zeros (their p is 0, and
    // whatever slot they were read from must not turn 0 * v into NaN); runs
    // after the loads of that tile have landed.
    auto zero_tail = [&](unsigned char *vt, int tile) {
        const int nvalid = k_hi - tile * BN;
        if (nvalid >= BN) return;
        for (int idx = tid; idx < (BN - nvalid) * CHK; idx += NT)
            *(uint4 *)(vt + (nvalid + idx / CHK) * ROWB + 16 * (idx % CHK)) = make_uint4(0, 0, 0, 0);
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
    auto s_tile = [&](const unsigned char *kt) {
        f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(kt + koff[0]), qf[0], mneg, 0, 0, 0);
#pragma unroll
        for (int t = 1; t < QT; t++)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(kt + koff[t]), qf[t], s, 0, 0, 0);
        return s;
    };
    // causal mask of tile n (absolute key of accumulator element j:
    // 32n + 8*(j/4) + 4*h2 + j%4) and the row maximum
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
        return max_xor32(mx);
    };
    // lazy move of the reference (scores and mx are relative to it); rescales
    // O and l, so it runs after the PV MFMAs issued before it
    auto move_ref = [&](f32x16 &s, float mx) {
        const bool need = mx > thr;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_ref = m_run == -INFINITY ? 0.f : m_run;
            const float shift = need ? mx : 0.f;
            const float m_new = m_ref + shift;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < DBLK; b++) oacc[b] *= alpha;
#pragma unroll
            for (int j = 0; j < 16; j++) {
                s[j] -= shift;
                mneg[j] = -m_new;
            }
            m_run = m_new;
            thr = kLazy;
        }
    };
    // p = 2^s rounded to bf16 (the B operands of the tile's 2 PV steps);
    // the row sum adds up the same rounded values, two at a time
    auto exp_tile = [&](const f32x16 &s, bf16x8 (&pf)[2]) {
#pragma unroll
        for (int j = 0; j < 16; j++) pf[j >> 3][j & 7] = (__bf16)__builtin_amdgcn_exp2f(s[j]);
        const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const bf16x2 pp = {pf[j >> 2][2 * (j & 3)], pf[j >> 2][2 * (j & 3) + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, l_run, false);
        }
    };
    // O^T += V^T P^T; step s2 covers keys 16*s2 + {4*h2 + 0..3, 8 + 4*h2 + 0..3}
    auto pv_tile = [&](const unsigned char *vt, const bf16x8 (&pf)[2]) {
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
#pragma unroll
            for (int b = 0; b < DBLK; b++) {
                const unsigned char *p0 = vt + s2 * 16 * ROWB + voff0[b];
                const unsigned char *p1 = vt + s2 * 16 * ROWB + voff1[b];
                i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p0);
                i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SGL_LDS i16x4 *)p1);
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 cat = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pf[s2],
                                                                 oacc[b], 0, 0, 0);
            }
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

    // ---- prologue: slot table, then K tiles 0..RING-1 and V tiles 0..RING-2
    // in the order of the stages -4..-1 they stand for
    fill(IC<2 * TABH / NT>{}, k_lo);
    __syncthreads();
    Off off0[NB], off1[NB];                          // offsets of tile j live in off[j % 2]
    auto offs = [&](auto i) -> Off (&)[NB] { return decltype(i)::value % 2 ? off1 : off0; };
    offsets(n0, off0);
    issue(k_pool, k_lds0, off0);
    offsets(n0 + 1, off1);
    issue(k_pool, k_lds1, off1);
    issue(v_pool, v_lds0, off0);
    offsets(n0 + 2, off0);
    issue(k_pool, k_lds2, off0);
    issue(v_pool, v_lds1, off1);
    offsets(n0 + 3, off1);
    issue(k_pool, k_lds3, off1);
    issue(v_pool, v_lds2, off0);
    vm_wait<6 * NB>();           // K tile n0
    lds_barrier();
    f32x16 s_cur = s_tile(k_lds0);
    move_ref(s_cur, n0 * BN + 31 > min_pos ? mask_max(s_cur, n0, std::true_type{})
                                           : mask_max(s_cur, n0, std::false_type{}));
    vm_wait<4 * NB>();           // V tile n0, K tile n0 + 1
    if (N == n0 + 1) zero_tail(v_lds0, n0);
    lds_barrier();

    // ---- stage n (R = n % RING): S^T(n+1) || p of tile n; PV of tile n ||
    // mask and max of tile n+1; then the loads of K tile n+RING and V tile
    // n+RING-1 into the ring slots that K tile n and V tile n-1 have left.
    // MASK: tile n+1 may cross the diagonal (a tile past the end is wholly
    // masked).
    auto stage = [&](const int n, auto r_tag, auto mask_tag) {
        constexpr int R = decltype(r_tag)::value;
        const f32x16 s_next = s_tile(kbuf(IC<R + 1>{}));
        bf16x8 pf[2];
        exp_tile(s_cur, pf);
        pv_tile(vbuf(IC<R>{}), pf);
        s_cur = s_next;
        const float mx = mask_max(s_cur, n + 1, mask_tag);
        // issue order: the K operand reads first, then each S^T MFMA with two
        // V^T reads and four VALU ops of the previous tile's softmax, then each
        // PV MFMA with the mask / maximum work of the next tile
        __builtin_amdgcn_sched_group_barrier(0x100, QT, 0);
#pragma unroll
        for (int t = 0; t < QT; t++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * DBLK / QT, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
#pragma unroll
        for (int t = 0; t < 2 * DBLK; t++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        move_ref(s_cur, mx);
        offsets(n + RING, offs(IC<R>{}));            // tile n+4; tile n+3's are in the other array
        issue(k_pool, kbuf(IC<R>{}), offs(IC<R>{}));
        issue(v_pool, vbuf(IC<R + RING - 1>{}), offs(IC<R + 1>{}));
        // K tile n+2 and V tile n+1 (issued RING-2 stages ago) have landed
        vm_wait<(RING - 2) * 2 * NB>();
        if (n + 2 == N) zero_tail(vbuf(IC<R + 1>{}), n + 1);
        lds_barrier();
    };
    // after stage 64m-1 of a long context, half (m+1) % 2 of the slot table
    // (chunk m-1, whose last look-up was at stage 64m-5) takes chunk m+1
    auto refill = [&](int n_done) {
        constexpr int SPC = TABH / BN;               // stages per chunk
        if (n_done % SPC == 0 && (n_done / SPC + 1) * TABH < k_hi)
            fill(IC<TABH / NT>{}, (n_done / SPC + 1) * TABH);
    };
    // stages whose look-ahead tile n+1 lies wholly at or below every row's
    // position need no mask; the loops run in groups of RING so that ring
    // positions are known at compile time
    // (a split's stages also stop before its last tile: the masked loop below
    // bounds every look-ahead by N)
    const int n_unmasked = min((min_pos >= 63 ? (min_pos - 63) / BN + 1 : 0) / RING * RING, (N - 1) / RING * RING);
    int n = n0;
    for (; n < n_unmasked; n += RING) {
        stage(n, IC<0>{}, std::false_type{});
        stage(n + 1, IC<1>{}, std::false_type{});
        stage(n + 2, IC<2>{}, std::false_type{});
        stage(n + 3, IC<3>{}, std::false_type{});
        refill(n + RING);
    }
    for (; n < N; n += RING) {
        stage(n, IC<0>{}, std::true_type{});
        if (n + 1 < N) stage(n + 1, IC<1>{}, std::true_type{});
        if (n + 2 < N) stage(n + 2, IC<2>{}, std::true_type{});
        if (n + 3 < N) stage(n + 3, IC<3>{}, std::true_type{});
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
