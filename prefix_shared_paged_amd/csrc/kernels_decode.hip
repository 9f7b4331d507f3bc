// kernels_decode.hip -- bf16 split-K decode attention for gfx950.
//
// Decode reads every K/V row of a request's context once and does little
// arithmetic per byte ("SGLang 深度拆解" (chenxutan.com) section 4.1: decode is
// memory-bound), so this kernel is built around keeping HBM busy.  On gfx950
// the achieved gather bandwidth grows with the number of waves resident per
// compute unit far more than with the bytes each wave has in flight (a wave
// resumes only when the slowest of its loads has returned), so every wave is
// kept small -- about 100 registers and 8-12 KiB of LDS:
//   - one work item per (KV head, key split, request or group);
//   - 16-key tiles: the K and V rows of a tile go straight from HBM into LDS
//     (global_load_lds_dwordx4, no register staging), each load instruction
//     covering four whole 256-byte rows, with non-temporal hints since every
//     row is read once.  The next tile's K loads are issued as soon as the
//     current K operands have been read, its V loads as soon as the current
//     V tile has been read;
//   - each row's 16-byte chunks are stored under an XOR swizzle (a bijection
//     of the row's low bits) so that the MFMA operand reads of K
//     (ds_read_b128, 16 rows x one chunk) and the transposed reads of V
//     (ds_read_b64_tr_b16) spread over the LDS banks.
// Per tile: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 keys on M, 16 query
// rows on N), the online-softmax update of p1 section 3.2 applied to the tile
// (fp32, base-2 exponentials with scale * log2(e) folded into one multiply),
// then O^T += V^T P^T with v_mfma_f32_16x16x16_bf16, whose B operand is exactly
// the S^T accumulator layout (lane: row, four consecutive keys), so P needs no
// lane exchange.  The split's state (m, l, unnormalised o) goes to the
// workspace; a merge kernel combines the splits of a request -- and for the
// cascade its group's prefix splits -- with the log-sum-exp rule.
//
// Work items: the flat call and the cascade suffix give the g = Hq/Hkv query
// heads of one request to a one-wave workgroup (16-row MFMA tiles, g <= 16),
// which keeps the most waves resident.  The cascade prefix stage gives all
// members x g query rows of a group to workgroups of up to four waves (16
// rows each) that share every prefix tile they load, so the shared prefix is
// read from HBM once per 64 query rows; it uses two tile buffers, since its
// work items are few and long.
#include <type_traits>

#include "common.h"
#include "decode_rows.h"
#include "decode_util.h"
#include "store_util.h"

namespace {

using namespace sgl_decode;

constexpr int TILE = 16;   // keys per tile
constexpr int PREFIX_DEPTH = 2;   // tile buffers of the cascade prefix stage
constexpr int kSlotTab = 2048;    // slot ids held in LDS at a time (longer splits refill)

// ---- work item of a split kernel ------------------------------------------------
// Workgroup id = ((item / 8) * n_rbg + rbg) * 8 + item % 8 with item = (split,
// set, KV head), split slowest: every request's first split is dispatched
// before any second one, so the waves that start last are the later (often
// partial) splits of long requests and the kernel's tail is short; and the
// first splits of a group's requests, which cover the shared prefix, run
// together.  rbg = which WPG row blocks of the item; consecutive ids differ in
// the KV head first, so the 8 XCDs see the 8 heads of one (split, set).
struct SplitItem {
    int kvh, s, first_req, n_members, row_base, nk;
    int64_t k0, ref_row;
    int64_t causal;   // kind 4: the row of member i sees keys <= causal + i; else -1
};

template <int WPG>
__device__ __forceinline__ bool split_item(const SplitArgs &a, int w, unsigned id, SplitItem &it) {
    const int n_rbg = (a.row_blocks + WPG - 1) / WPG;
    const unsigned rest = id >> 3;
    const int rbg = (int)(rest % (unsigned)n_rbg);
    const int64_t item = (int64_t)(rest / (unsigned)n_rbg) * 8 + (id & 7);
    const int kvh = (int)(item % a.Hkv);
    const int64_t t_ = item / a.Hkv;
    const int64_t set64 = t_ % a.n_sets;
    const int s = (int)(t_ / a.n_sets);
    if (s >= a.max_splits) return false;
    if (set64 >= a.n_sets) return false;
    const int set = (int)set64;
    const int g = a.Hq / a.Hkv;

    // which rows, which keys (uniform over the workgroup)
    int first_req, n_members;
    int64_t lo, hi, ref_row, chunk = a.chunk;
    it.causal = -1;
    if (a.kind == 4) {
        // small-q extend: the members are the request's new tokens
        const int64_t t0 = a.q_off[set], E = a.q_off[set + 1] - t0;
        const int64_t P = a.prefix_lens[set];
        if (E <= 0 || t0 < 0 || P < 0) return false;
        first_req = (int)t0;
        n_members = (int)E;
        lo = 0;
        hi = P + E;
        chunk = verify_chunk(hi, a.n_spl);
        ref_row = a.req_rows[set];
        it.causal = P;
    } else if (a.kind == 1) {
        first_req = a.group_ptr[set];
        n_members = a.group_ptr[set + 1] - first_req;
        if (n_members <= 0 || first_req < 0 || first_req + n_members > a.batch) return false;
        const int64_t P = a.group_prefix_len[set];
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
            const int64_t P =
                a.suffix_lo ? a.suffix_lo[set] : a.group_prefix_len[wave_find_group(a.group_ptr, a.G, set)];
            lo = P < 0 ? 0 : (P > L ? L : P);
        }
        hi = L;
    }
    if (n_members * g <= rbg * WPG * 16) return false;    // no rows left for this workgroup
    if (ref_row < 0 || ref_row >= a.num_rows) return false;
    if (hi > a.row_stride) hi = a.row_stride;
    const int64_t n_split = ceil_div64(hi - lo, chunk);
    if (s >= n_split || s >= a.part.S) return false;
    it.kvh = kvh;
    it.s = s;
    it.first_req = first_req;
    it.n_members = n_members;
    it.row_base = (rbg * WPG + w) * 16;
    it.k0 = lo + (int64_t)s * chunk;
    it.nk = (int)((it.k0 + chunk < hi ? it.k0 + chunk : hi) - it.k0);
    it.ref_row = ref_row;
    return true;
}

// WPG waves per workgroup share each K/V tile in LDS: the loads of a tile
// are split among them (each issues NI/WPG of the K and of the V load
// instructions) and every wave computes its own 16 query rows against the
// whole tile.  DEPTH LDS buffers per tile ring: with 1, tile n+1's K loads go
// out once tile n's K operands are read and its V loads once tile n's V is
// read; with more, DEPTH-1 tiles are in flight while one is computed.
//
// The work item is that of workgroup id (see split_item); k_lds and v_lds
// hold DEPTH tiles each, slot_lds min(chunk, kSlotTab) slot ids (kSlotTab
// for kind 4).
template <int D, int DEPTH, int WPG>
__device__ __forceinline__ void bf16_split(const SplitArgs &a, unsigned id, unsigned char *k_lds,
                                           unsigned char *v_lds, int32_t *slot_lds) {
    constexpr int QT = D / 32;          // MFMA k-steps over head_dim
    constexpr int DB = D / 16;          // 16-dim output blocks
    constexpr int ROWB = 2 * D;         // bytes of one K/V row of one head
    constexpr int CHK = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / CHK;       // rows per direct-load instruction (1 KiB)
    constexpr int NI = TILE / RPI;      // direct-load instructions per K or V tile
    static_assert(NI % WPG == 0, "each wave issues the same number of loads");
    static_assert(DEPTH >= 1 && DEPTH <= 4, "ring depth");
    constexpr int NIW = NI / WPG;       // K (and V) load instructions per wave per tile
    constexpr int TB = TILE * ROWB;   // tile t of the split lives in ring buffer t % DEPTH

    const int lane = threadIdx.x & 63;
    const int w = WPG > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    auto wg_barrier = [&]() {
        if (WPG > 1) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };

    SplitItem it;
    if (!split_item<WPG>(a, w, id, it)) return;
    const int kvh = it.kvh, s = it.s, g = a.Hq / a.Hkv;
    const int first_req = it.first_req, n_members = it.n_members;
    const int64_t k0 = it.k0, ref_row = it.ref_row;
    const int nk = it.nk;
    const int row_base = it.row_base;               // first group row of this wave
    const int rows = n_members * g - row_base;      // may be <= 0: the wave still loads

    // slot ids of the split's keys [pb, pb + kSlotTab) in LDS (one part unless
    // the split is longer than the table)
    const int32_t *row = a.r2t + ref_row * a.row_stride + k0;
    auto fill_slots = [&](int pb) {
        const int cnt = min(kSlotTab, nk - pb);
        for (int j = threadIdx.x; j < cnt; j += 64 * WPG) slot_lds[j] = safe_slot(row[pb + j], a.num_slots);
    };
    fill_slots(0);

    const __bf16 *q = (const __bf16 *)a.q;
    const char *kp = (const char *)a.k_pool + kvh * D * 2;
    const char *vp = (const char *)a.v_pool + kvh * D * 2;
    const int64_t rowstride_el = (int64_t)a.Hkv * D;
    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand: lane (row n16, kq) holds dims 32t + 8kq + i in step t --
    bf16x8 qf[QT];
    {
        const int rho = n16 < rows ? n16 : 0;
        const int rr = row_base + rho < n_members * g ? row_base + rho : 0;
        const int req = first_req + rr / g;
        const int h = kvh * g + rr % g;
        const __bf16 *src = q + ((int64_t)req * a.Hq + h) * D + 8 * kq;
#pragma unroll
        for (int t = 0; t < QT; t++) qf[t] = ld_q(src + 32 * t);
        if (n16 >= rows)
#pragma unroll
            for (int t = 0; t < QT; t++) qf[t] = bf16x8{};
    }

    // ---- per-lane constants of the loads and LDS reads --------------------------
    // direct load instruction ii: lane -> row ii*RPI + lane/CHK of the tile, LDS
    // position lane%CHK, which holds chunk (lane%CHK) ^ swz(row).  This wave
    // issues instructions ii = w + WPG*u of the K tile and of the V tile.
    const int lrow0 = lane / CHK;
    int lrow[NIW], lchk[NIW];
#pragma unroll
    for (int u = 0; u < NIW; u++) {
        const int ii = w + WPG * u;
        lrow[u] = ii * RPI + lrow0;
        lchk[u] = 16 * ((lane % CHK) ^ swz<D>(lrow[u]));
    }
    // K operand of step t: lane (key n16, kq) reads chunk 4t + kq of row n16
    const int ksw = swz<D>(n16);
    const int kbase = n16 * ROWB;
    // V^T read of dim block db: lane (r4, qq) of group kq reads 4 dims of row
    // (key) 4kq + r4; the transposed result gives lane (dim, kq) keys 4kq..4kq+3
    const int r4 = n16 >> 2, qq = n16 & 3;
    const int vr = kq * 4 + r4;
    const int vsw = swz<D>(vr);
    const int vbase = vr * ROWB + 8 * (qq & 1);

    __syncthreads();   // slot table visible

    // keys of the current slot-table part: [pbase, pbase + nkp) of the split
    int pbase = 0, nkp = min(kSlotTab, nk);
    // small-q extend: this lane's row sees split keys <= clim
    const int clim = it.causal >= 0 ? (int)(it.causal + (row_base + n16) / g - k0) : 0x7fffffff;

    // This wave's loads of tile n of the part (keys past its end repeat its
    // last key, so every address is a real row of the context; their scores
    // are masked)
    auto issue = [&](int n, const char *pool, unsigned char *dst) {
#pragma unroll
        for (int u = 0; u < NIW; u++) {
            const int kk = min(n * TILE + lrow[u], nkp - 1);
            const char *src = pool + (int64_t)slot_lds[kk] * rowstride_el * 2 + lchk[u];
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                             (SGL_LDS void *)(dst + (w + WPG * u) * 1024), 16, 0, 2 /* nt */);
        }
    };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float qscale = a.scale * kLog2e;

    // S^T = K Q^T of one tile: lane (row n16, kq) gets keys 4kq + j
    auto s_tile = [&](const unsigned char *kb) {
        const uint32_t b = lds_addr(kb) + kbase;
        uint32_t ad[QT];
#pragma unroll
        for (int t = 0; t < QT; t++) ad[t] = b + 16 * ((4 * t + kq) ^ ksw);
        bf16x8 kf[QT];
        lds_read_b128(kf, ad);
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < QT; t++) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t], qf[t], sacc, 0, 0, 0);
        return sacc;
    };
    // online softmax of the row over tile n, then O^T += V^T P^T
    auto pv_tile = [&](int n, const f32x4 &sacc, const unsigned char *vb) {
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int kidx = pbase + n * TILE + kq * 4 + j;
            const float x = kidx < nk && kidx <= clim ? sacc[j] * qscale : -INFINITY;
            sv[j] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference m_run moves only when a row's tile maximum exceeds it
        // by more than 2^8 (always on the first tile), so most tiles skip the
        // rescale of O and l; p = 2^(s - m_run) <= 2^8 stays exact in fp32 and
        // in range for bf16, and o / l does not depend on the reference.
        const bool move = mx > m_run + 8.f;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? mx : m_run;        // finite: every tile has a valid key
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
            m_run = m_new;
        }
        // a row with no visible key so far keeps m_run = -inf (its scores are
        // all -inf, and 2^(-inf - 0) = 0)
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        bf16x4 pf;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float pj = __builtin_amdgcn_exp2f(sv[j] - m_use);
            l_run += pj;
            pf[j] = (__bf16)pj;
        }
        // 16 dims x 16 keys per MFMA
        const uint32_t b = lds_addr(vb) + vbase;
        uint32_t ad[DB];
#pragma unroll
        for (int db = 0; db < DB; db++) ad[db] = b + 16 * ((2 * db + (qq >> 1)) ^ vsw);
        i16x4 vt[DB];
        lds_read_tr16(vt, ad);
#pragma unroll
        for (int db = 0; db < DB; db++)
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[db], __builtin_bit_cast(i16x4, pf), oacc[db],
                                                                 0, 0, 0);
    };

    for (;;) {
        const int N = (nkp + TILE - 1) / TILE;      // tiles of this part, >= 1
        if constexpr (DEPTH == 1) {
            issue(0, kp, k_lds);
            issue(0, vp, v_lds);
            for (int n = 0; n < N; n++) {
                vm_wait<0>();                        // this wave's loads of tile n have landed
                wg_barrier();                        // ... and every wave's
                const f32x4 sacc = s_tile(k_lds);
                if (n + 1 < N) {
                    lgkm_wait0();
                    wg_barrier();                    // every wave has read the K tile
                    issue(n + 1, kp, k_lds);
                }
                pv_tile(n, sacc, v_lds);
                if (n + 1 < N) {
                    lgkm_wait0();
                    wg_barrier();                    // every wave has read the V tile
                    issue(n + 1, vp, v_lds);
                }
            }
        } else {
            // DEPTH-1 tiles stay in flight while one is computed
            for (int t = 0; t < DEPTH && t < N; t++) {
                issue(t, kp, k_lds + (t % DEPTH) * TB);
                issue(t, vp, v_lds + (t % DEPTH) * TB);
            }
            for (int n = 0; n < N; n++) {
                const int ahead = min(DEPTH - 1, N - 1 - n);   // tiles issued after tile n
                // this wave's loads of tile n have landed when at most ahead * 2 * NIW remain
                if (ahead >= 3) vm_wait<3 * 2 * NIW>();
                else if (ahead == 2) vm_wait<2 * 2 * NIW>();
                else if (ahead == 1) vm_wait<2 * NIW>();
                else vm_wait<0>();
                wg_barrier();
                unsigned char *kb = k_lds + (n % DEPTH) * TB;
                unsigned char *vb = v_lds + (n % DEPTH) * TB;
                pv_tile(n, s_tile(kb), vb);
                if (n + DEPTH < N) {
                    lgkm_wait0();
                    wg_barrier();                    // every wave is done with this buffer
                    issue(n + DEPTH, kp, kb);
                    issue(n + DEPTH, vp, vb);
                }
            }
        }
        pbase += kSlotTab;
        if (pbase >= nk) break;
        // next part of a long split: every wave is done with the table and
        // the tile buffers (no load is in flight); refill the table
        __syncthreads();
        fill_slots(pbase);
        nkp = min(kSlotTab, nk - pbase);
        __syncthreads();
    }

    // ---- write the split's state ---------------------------------------------
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 >= rows) return;
    const int req = first_req + (row_base + n16) / g;
    const int h = kvh * g + (row_base + n16) % g;
    const int64_t idx = ((int64_t)req * a.part.S + s) * a.Hq + h;
    float *op = a.part.o + idx * D;
#pragma unroll
    for (int db = 0; db < DB; db++) *(f32x4 *)(op + db * 16 + kq * 4) = oacc[db];
    if (kq == 0) *(float2 *)(a.part.ml + idx * 2) = make_float2(m_run, l);
}

// =============================================================================
// FP8 (e4m3fn) KV cache.  The pools hold one byte per element and one fp32
// factor per KV head for K and for V; code c of head kv stands for
// decode(c) * scale[kv].  Every e4m3fn value is exact in bf16, so the tiles
// are widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, two codes per
// instruction, factor 1) and the bf16 MFMAs of the kernel above do the rest;
// the K factor joins the score scale and the V factor multiplies the split's
// output.  A tile holds 32 keys, the same 4 KiB per pool as a bf16 tile of 16
// keys at D = 128:
//   - S^T = K Q^T as two 16-key MFMA blocks.  Block b's row m is tile key
//     8 (m / 4) + 4 b + m % 4, so that the accumulators give lane (row, kq)
//     the 8 consecutive keys 8 kq .. 8 kq + 7, which is the B operand layout of
//     the 32-key PV MFMA: P needs no lane exchange.
//   - The head dims are split into four contiguous quarters, one per lane
//     group kq (the order of a dot product's terms is free as long as Q and K
//     agree), so a lane reads whole 16-byte chunks of K rows.
//   - O^T += V^T P^T with v_mfma_f32_16x16x32_bf16; its A operand (lane: one
//     dim, 8 consecutive keys) comes from ds_read_b64_tr_b8, which hands lane
//     (j, group G) byte k of the 8 rows addressed by its group, column j.
// =============================================================================
constexpr int TILE8 = 32;   // keys per fp8 tile

// The work item is that of workgroup id (see split_item); k_lds and v_lds
// hold DEPTH tiles each, slot_lds chunk slot ids.
template <int D, int DEPTH, int WPG>
__device__ __forceinline__ void fp8_split(const SplitArgs &a, unsigned id, unsigned char *k_lds,
                                          unsigned char *v_lds, int32_t *slot_lds) {
    constexpr int QT = D / 32;          // MFMA k-steps over head_dim
    constexpr int DB = D / 16;          // 16-dim output blocks
    constexpr int ROWB = D;             // bytes of one K/V row of one head
    constexpr int CHK = D / 16;         // 16-byte chunks per row
    constexpr int RPI = 64 / CHK;       // rows per direct-load instruction (1 KiB)
    constexpr int NI = TILE8 / RPI;     // direct-load instructions per K or V tile
    static_assert(NI % WPG == 0, "each wave issues the same number of loads");
    static_assert(DEPTH >= 1 && DEPTH <= 4, "ring depth");
    constexpr int NIW = NI / WPG;
    constexpr int TB = TILE8 * ROWB;
    constexpr int KCH = D / 64;         // K chunks per lane per 16-key block (a quarter row)

    const int lane = threadIdx.x & 63;
    const int w = WPG > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    auto wg_barrier = [&]() {
        if (WPG > 1) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };

    SplitItem it;
    if (!split_item<WPG>(a, w, id, it)) return;
    const int kvh = it.kvh, s = it.s, g = a.Hq / a.Hkv;
    const int first_req = it.first_req, n_members = it.n_members;
    const int nk = it.nk;
    const int N = (nk + TILE8 - 1) / TILE8;         // tiles, >= 1
    const int row_base = it.row_base;
    const int rows = n_members * g - row_base;      // may be <= 0: the wave still loads

    const int32_t *row = a.r2t + it.ref_row * a.row_stride + it.k0;
    for (int j = threadIdx.x; j < nk; j += 64 * WPG) slot_lds[j] = safe_slot(row[j], a.num_slots);

    const __bf16 *q = (const __bf16 *)a.q;
    const unsigned char *kp = (const unsigned char *)a.k_pool + kvh * D;
    const unsigned char *vp = (const unsigned char *)a.v_pool + kvh * D;
    const int64_t rowstride = (int64_t)a.Hkv * D;   // bytes per slot
    const int n16 = lane & 15, kq = lane >> 4;

    // ---- Q^T operand: lane (row n16, kq) holds dims kq*D/4 + 8t + i in step t --
    bf16x8 qf[QT];
    {
        const int rho = n16 < rows ? n16 : 0;
        const int rr = row_base + rho < n_members * g ? row_base + rho : 0;
        const int req = first_req + rr / g;
        const int h = kvh * g + rr % g;
        const __bf16 *src = q + ((int64_t)req * a.Hq + h) * D + kq * (D / 4);
#pragma unroll
        for (int t = 0; t < QT; t++) qf[t] = ld_q(src + 8 * t);
        if (n16 >= rows)
#pragma unroll
            for (int t = 0; t < QT; t++) qf[t] = bf16x8{};
    }

    // ---- per-lane constants of the loads and LDS reads --------------------------
    const int lrow0 = lane / CHK;
    int lrow[NIW], lchk[NIW];
#pragma unroll
    for (int u = 0; u < NIW; u++) {
        const int ii = w + WPG * u;
        lrow[u] = ii * RPI + lrow0;
        lchk[u] = 16 * ((lane % CHK) ^ swz8<D>(lrow[u]));
    }
    // K block b: lane (n16, kq) reads the chunks KCH*kq .. of tile row kr[b]
    int kbase[2], ksw[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const int kr = 8 * (n16 >> 2) + 4 * b + (n16 & 3);
        kbase[b] = kr * ROWB;
        ksw[b] = swz8<D>(kr);
    }
    // V^T of dim block db: lane (n16, kq) addresses row 8kq + n16/2, half n16%2
    // of chunk db; the result gives lane (dim 16db + n16, kq) keys 8kq .. 8kq+7
    const int vr = 8 * kq + (n16 >> 1);
    const int vsw = swz8<D>(vr);
    const int vbase = vr * ROWB + 8 * (n16 & 1);

    __syncthreads();   // slot table visible

    auto issue = [&](int n, const unsigned char *pool, unsigned char *dst) {
#pragma unroll
        for (int u = 0; u < NIW; u++) {
            const int kk = min(n * TILE8 + lrow[u], nk - 1);
            const unsigned char *src = pool + (int64_t)slot_lds[kk] * rowstride + lchk[u];
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                             (SGL_LDS void *)(dst + (w + WPG * u) * 1024), 16, 0, 2 /* nt */);
        }
    };

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float qscale = a.scale * kLog2e * a.k_scale[kvh];

    // S^T = K Q^T of one tile, two 16-key blocks
    auto s_tile = [&](const unsigned char *kb, f32x4 (&sacc)[2]) {
        const uint32_t b0 = lds_addr(kb);
        uint32_t ad[2 * KCH];
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int c = 0; c < KCH; c++) ad[b * KCH + c] = b0 + kbase[b] + 16 * ((KCH * kq + c) ^ ksw[b]);
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
    };
    // online softmax of the row over tile n, then O^T += V^T P^T
    auto pv_tile = [&](int n, const f32x4 (&sacc)[2], const unsigned char *vb) {
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = n * TILE8 + 8 * kq + 4 * b + j < nk ? sacc[b][j] * qscale : -INFINITY;
                sv[4 * b + j] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // lazy reference maximum, as in split_bf16_kernel
        const bool move = mx > m_run + 8.f;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
            m_run = m_new;
        }
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float pj = __builtin_amdgcn_exp2f(sv[j] - m_run);
            l_run += pj;
            pf[j] = (__bf16)pj;
        }
        const uint32_t b = lds_addr(vb) + vbase;
        uint32_t ad[DB];
#pragma unroll
        for (int db = 0; db < DB; db++) ad[db] = b + 16 * (db ^ vsw);
        i32x2 vt[DB];
        lds_read_tr8(vt, ad);
#pragma unroll
        for (int db = 0; db < DB; db++)
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(vt[db][0], vt[db][1]), pf,
                                                                oacc[db], 0, 0, 0);
    };

    if constexpr (DEPTH == 1) {
        issue(0, kp, k_lds);
        issue(0, vp, v_lds);
        for (int n = 0; n < N; n++) {
            vm_wait<0>();
            wg_barrier();
            f32x4 sacc[2];
            s_tile(k_lds, sacc);
            if (n + 1 < N) {
                wg_barrier();                            // every wave has read the K tile
                issue(n + 1, kp, k_lds);
            }
            pv_tile(n, sacc, v_lds);
            if (n + 1 < N) {
                wg_barrier();                            // every wave has read the V tile
                issue(n + 1, vp, v_lds);
            }
        }
    } else {
        for (int t = 0; t < DEPTH && t < N; t++) {
            issue(t, kp, k_lds + (t % DEPTH) * TB);
            issue(t, vp, v_lds + (t % DEPTH) * TB);
        }
        for (int n = 0; n < N; n++) {
            const int ahead = min(DEPTH - 1, N - 1 - n);
            if (ahead >= 3) vm_wait<3 * 2 * NIW>();
            else if (ahead == 2) vm_wait<2 * 2 * NIW>();
            else if (ahead == 1) vm_wait<2 * NIW>();
            else vm_wait<0>();
            wg_barrier();
            unsigned char *kb = k_lds + (n % DEPTH) * TB;
            unsigned char *vb = v_lds + (n % DEPTH) * TB;
            f32x4 sacc[2];
            s_tile(kb, sacc);
            pv_tile(n, sacc, vb);
            if (n + DEPTH < N) {
                wg_barrier();                            // every wave is done with this buffer
                issue(n + DEPTH, kp, kb);
                issue(n + DEPTH, vp, vb);
            }
        }
    }

    // ---- write the split's state (o carries the V factor) --------------------
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 >= rows) return;
    const float vscale = a.v_scale[kvh];
    const int req = first_req + (row_base + n16) / g;
    const int h = kvh * g + (row_base + n16) % g;
    const int64_t idx = ((int64_t)req * a.part.S + s) * a.Hq + h;
    float *op = a.part.o + idx * D;
#pragma unroll
    for (int db = 0; db < DB; db++) *(f32x4 *)(op + db * 16 + kq * 4) = oacc[db] * vscale;
    if (kq == 0) *(float2 *)(a.part.ml + idx * 2) = make_float2(m_run, l);
}

// a.store.n_wg > 0 (a cascade prefix stage): the first a.store.n_wg
// workgroups run the decode store of the call's current tokens and the
// suffix starts instead (the prefix items read positions below every
// request's group prefix length, which stays below its current token's
// position, and the suffix stage and the merge that read the token and the
// starts are later launches); the split items follow, numbered from 0, and
// n_wg is a multiple of 8, so each keeps its XCD.
template <int D, int DEPTH, int WPG>
__global__ void __launch_bounds__(64 * WPG) split_bf16_kernel(SplitArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[DEPTH * TILE * 2 * D];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[DEPTH * TILE * 2 * D];
    extern __shared__ int32_t slot_lds[];  // [min(chunk, kSlotTab)]
    const unsigned nst = (unsigned)a.store.n_wg;
    if (blockIdx.x < nst) {
        decode_store_job<2, false>(a.store, blockIdx.x, nst);
        return;
    }
    bf16_split<D, DEPTH, WPG>(a, blockIdx.x - nst, k_lds, v_lds, slot_lds);
}

template <int D, int DEPTH, int WPG>
__global__ void __launch_bounds__(64 * WPG) split_fp8_kernel(SplitArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[DEPTH * TILE8 * D];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[DEPTH * TILE8 * D];
    extern __shared__ int32_t slot_lds[];  // [chunk]
    const unsigned nst = (unsigned)a.store.n_wg;
    if (blockIdx.x < nst) {                  // bf16 inputs (the launcher checks)
        decode_store_job<2, true>(a.store, blockIdx.x, nst);
        return;
    }
    fp8_split<D, DEPTH, WPG>(a, blockIdx.x - nst, k_lds, v_lds, slot_lds);
}

// ---- cascade: prefix and suffix stages in one grid ----------------------------
// The grid holds three ranges of workgroups: suffix-stage items of the first
// head split rounds (rows_split over four KV heads), then the prefix-stage
// items (bf16_split / fp8_split, four waves sharing a ring of four tiles: up
// to 64 query rows of a group per KV head), then the suffix items of the
// remaining rounds.  Every range holds a multiple of 8 workgroups, so each
// item lands on the XCD it would have in a launch of its own.  The stages
// read only the pools and write disjoint state buffers, so nothing orders
// them.  In one grid the call makes one launch fewer and neither stage waits
// for the other to drain: on the 256-request decode workload the suffix
// items (1 MiB each) go first and the prefix items, four times smaller, fill
// the compute units as the suffix items run out, which shortens the tail.
// The suffix grid is sized by max_seq_len, so its late rounds are mostly
// empty workgroups when suffixes are shorter than that; dispatching those
// after the prefix items keeps them from delaying real work.
// Both stages fit one LDS budget: 32 KiB of tiles (two 16 KiB suffix tiles
// or 2 x 4 prefix tiles of 4 KiB) and a slot table.
template <int D, bool FP8>
__global__ void __launch_bounds__(256) cascade_split_kernel(SplitArgs pa, SplitArgs sa, unsigned n_head,
                                                            unsigned n_pre) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    constexpr int PTB = FP8 ? TILE8 * D : TILE * 2 * D;             // prefix tile bytes
    constexpr int STB = (FP8 ? 32 : 16) * kRowsHeads * D * (FP8 ? 1 : 2);   // suffix tile bytes
    static_assert(8 * PTB == 2 * STB, "one LDS budget");
    const unsigned id = blockIdx.x;
    if (id < n_head || id - n_head >= n_pre) {
        const unsigned sid = id < n_head ? id : id - n_pre;
        rows_split<D, FP8, kRowsHeads>(sa, (int)sid, (int)threadIdx.x, dyn_lds, dyn_lds + STB,
                                        (int32_t *)(dyn_lds + 2 * STB));
    } else {
        int32_t *slots = (int32_t *)(dyn_lds + 8 * PTB);
        if constexpr (FP8) fp8_split<D, 4, 4>(pa, id - n_head, dyn_lds, dyn_lds + 4 * PTB, slots);
        else bf16_split<D, 4, 4>(pa, id - n_head, dyn_lds, dyn_lds + 4 * PTB, slots);
    }
}

// ---- cascade: balanced suffix runs, then the prefix items, in one grid ---------
// The suffixes of all requests laid end to end, every workgroup of a head
// group taking an equal run of them (balanced_run, 4 KV heads per
// workgroup: all of them resident at once, so the grid does not drain as
// split items of suffix-long work would), and behind them the prefix items
// (bf16_split, four waves sharing a ring of four tiles), which take the
// compute units as the runs finish.  The LDS budget is cascade_split_kernel's.
// sa is the first argument: balanced_run reads it through the kernarg pointer.
template <int D, bool FP8>
__global__ void __launch_bounds__(256, 4) cascade_balanced_kernel(SplitArgs sa, SplitArgs pa, unsigned n_bal) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    constexpr int PTB = FP8 ? TILE8 * D : TILE * 2 * D;                 // prefix tile bytes
    constexpr int STB = (FP8 ? 32 : 16) * kRowsHeads * D * (FP8 ? 1 : 2);   // suffix tile bytes
    static_assert(8 * PTB == 2 * STB, "one LDS budget");
    const unsigned id = blockIdx.x;
    if (id < n_bal) {
        const unsigned ng = (unsigned)(sa.Hkv / kRowsHeads);
        balanced_run<D, FP8, kRowsHeads>((KArgs)__builtin_amdgcn_kernarg_segment_ptr(), id / ng, (int)(id % ng),
                                         dyn_lds, dyn_lds + STB, (int32_t *)(dyn_lds + 2 * STB));
    } else {
        int32_t *slots = (int32_t *)(dyn_lds + 8 * PTB);
        if constexpr (FP8) fp8_split<D, 4, 4>(pa, id - n_bal, dyn_lds, dyn_lds + 4 * PTB, slots);
        else bf16_split<D, 4, 4>(pa, id - n_bal, dyn_lds, dyn_lds + 4 * PTB, slots);
    }
}

}  // namespace

// bf16 cascade: one grid of the balanced suffix runs (sa.sk_wgs per head
// group of 4 KV heads) and the prefix items.  The current tokens, the suffix
// starts and the plan (SuffixStartArgs::plan) must already be written.
int launch_cascade_balanced(const SplitArgs &pa0, const SplitArgs &sa, bool fp8, hipStream_t st) {
    if (pa0.kind != 1 || sa.kind != 2 || !sa.suffix_lo || !sa.sk_plan || sa.sk_wgs < 1 || sa.part.S != 1)
        return SGL_ERR_INVALID;
    if (pa0.D != sa.D || pa0.Hkv != sa.Hkv || pa0.Hq != sa.Hq) return SGL_ERR_INVALID;
    if (sa.D != 128 || sa.Hkv % kRowsHeads != 0 || sa.Hkv > 16 || sa.Hq / sa.Hkv > 16) return SGL_ERR_UNSUPPORTED;
    const int tk = fp8 ? TILE8 : TILE;
    if (pa0.chunk % tk != 0 || sa.chunk % tk != 0) return SGL_ERR_INVALID;
    if (fp8 && (!sa.k_scale || !sa.v_scale || !pa0.k_scale || !pa0.v_scale)) return SGL_ERR_INVALID;
    SplitArgs pa = pa0;
    pa.row_blocks = (pa.max_members * (pa.Hq / pa.Hkv) + 15) / 16;
    const int64_t n_rbg = (pa.row_blocks + 3) / 4;
    const int64_t p_items = (int64_t)pa.n_sets * pa.max_splits * pa.Hkv;
    const int64_t n_pre = ceil_div64(p_items, 8) * 8 * n_rbg;
    const int64_t n_bal = (int64_t)sa.sk_wgs * (sa.Hkv / kRowsHeads);
    if (n_pre + n_bal > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const int64_t p_slots = fp8 ? pa.chunk : min(pa.chunk, kSlotTab);
    const size_t dyn = 32768 + (size_t)(p_slots > sa.chunk ? p_slots : sa.chunk) * sizeof(int32_t);
    if (fp8)
        hipLaunchKernelGGL((cascade_balanced_kernel<128, true>), dim3((unsigned)(n_pre + n_bal)), dim3(256), dyn, st,
                           sa, pa, (unsigned)n_bal);
    else
        hipLaunchKernelGGL((cascade_balanced_kernel<128, false>), dim3((unsigned)(n_pre + n_bal)), dim3(256), dyn, st,
                           sa, pa, (unsigned)n_bal);
    return hip_status(hipGetLastError());
}

int launch_cascade_split(const SplitArgs &pa0, const SplitArgs &sa, int32_t head_rounds, bool fp8, hipStream_t st) {
    if (pa0.kind != 1 || sa.kind != 2) return SGL_ERR_INVALID;
    if (pa0.D != 128 || sa.D != 128 || pa0.Hkv != sa.Hkv || pa0.Hq != sa.Hq) return SGL_ERR_UNSUPPORTED;
    if (sa.Hkv % kRowsHeads != 0 || sa.Hkv > 16 || sa.Hq / sa.Hkv > 16) return SGL_ERR_UNSUPPORTED;
    const int tk = fp8 ? TILE8 : TILE;
    if (pa0.chunk % tk != 0 || sa.chunk % tk != 0 || sa.xcd_block < 1) return SGL_ERR_INVALID;
    if (fp8 && (!sa.k_scale || !sa.v_scale || !pa0.k_scale || !pa0.v_scale)) return SGL_ERR_INVALID;
    SplitArgs pa = pa0;
    pa.row_blocks = (pa.max_members * (pa.Hq / pa.Hkv) + 15) / 16;
    const int64_t n_rbg = (pa.row_blocks + 3) / 4;
    const int64_t p_items = (int64_t)pa.n_sets * pa.max_splits * pa.Hkv;
    const int64_t n_pre = ceil_div64(p_items, 8) * 8 * n_rbg;
    // suffix workgroups per split round, as rows_split numbers them
    const int rb = sa.xcd_block;
    const int64_t n_v = (int64_t)sa.n_sets * (sa.Hkv / kRowsHeads);
    const int64_t per_round = sa.n_sets > 0 ? 8 * (((n_v + rb - 1) / rb + 7) / 8) * rb : 0;
    const int64_t n_suf = per_round * sa.max_splits;
    const int64_t head = head_rounds < 0 ? 0 : (head_rounds > sa.max_splits ? sa.max_splits : head_rounds);
    const int64_t n_head = per_round * head;
    if (n_pre + n_suf == 0) return SGL_OK;
    if (n_pre + n_suf > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const int64_t p_slots = fp8 ? pa.chunk : min(pa.chunk, kSlotTab);
    const size_t dyn = 32768 + (size_t)(p_slots > sa.chunk ? p_slots : sa.chunk) * sizeof(int32_t);
    const dim3 grid((unsigned)(n_pre + n_suf)), block(256);
    if (fp8)
        hipLaunchKernelGGL((cascade_split_kernel<128, true>), grid, block, dyn, st, pa, sa, (unsigned)n_head,
                           (unsigned)n_pre);
    else
        hipLaunchKernelGGL((cascade_split_kernel<128, false>), grid, block, dyn, st, pa, sa, (unsigned)n_head,
                           (unsigned)n_pre);
    return hip_status(hipGetLastError());
}

// The decode store carried by a prefix-stage launch: its workgroup count for
// `threads`-thread workgroups (0 when there is none); rejects a store the
// kernels do not carry.
static int carried_store(SplitArgs &a, bool fp8, int threads) {
    const bool any = a.store.n_tokens > 0 || a.store.ss.lo;
    a.store.n_wg = 0;
    if (!any) return SGL_OK;
    if (a.kind != 1 || a.store.fp8 != (fp8 ? 1 : 0) || (fp8 && a.store.elt != 2)) return SGL_ERR_INVALID;
    if (fp8 && a.store.n_tokens > 0 && (!a.store.k_scale || !a.store.v_scale)) return SGL_ERR_INVALID;
    a.store.n_wg = decode_store_wgs(a.store, threads);
    return SGL_OK;
}

int launch_split_bf16(const SplitArgs &a0, hipStream_t st) {
    if ((a0.n_sets == 0 || a0.max_splits == 0) && a0.store.n_tokens == 0 && !a0.store.ss.lo) return SGL_OK;
    if (a0.chunk % TILE != 0) return SGL_ERR_INVALID;
    SplitArgs a = a0;
    const bool multi = a.kind == 1 || a.kind == 4;   // several query rows per (set, KV head)
    const int rows = (multi ? a.max_members : 1) * (a.Hq / a.Hkv);
    a.row_blocks = (rows + 15) / 16;
    // The flat and suffix calls have many short work items: one wave per
    // workgroup and one buffer keep the most waves resident.  The prefix
    // stage (and a small-q extend) has up to 4 row blocks (64 query rows)
    // per KV head: the row blocks share each tile, and a ring of PREFIX_DEPTH
    // buffers keeps several tiles in flight per workgroup.
    int wpg = 1;
    if (multi) wpg = a.row_blocks >= 3 ? 4 : a.row_blocks;
    if (a.D == 64 && wpg > 2) wpg = 2;               // 2 load instructions per 64-dim tile
    const int n_rbg = (a.row_blocks + wpg - 1) / wpg;
    const int64_t items = (int64_t)a.n_sets * a.max_splits * a.Hkv;
    int rc = carried_store(a, false, 64 * wpg);
    if (rc != SGL_OK) return rc;
    const int64_t n_wg = ceil_div64(items, 8) * 8 * n_rbg + a.store.n_wg;
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const size_t dyn = (size_t)(a.kind == 4 ? kSlotTab : min(a.chunk, kSlotTab)) * sizeof(int32_t);
    const dim3 grid((unsigned)n_wg), block(64 * wpg);
#define SGL_SPLIT(DD, DP, W) hipLaunchKernelGGL((split_bf16_kernel<DD, DP, W>), grid, block, dyn, st, a)
    if (a.D == 128) {
        if (wpg == 1) { if (a.kind == 1) SGL_SPLIT(128, PREFIX_DEPTH, 1); else SGL_SPLIT(128, 1, 1); }
        else if (wpg == 2) SGL_SPLIT(128, PREFIX_DEPTH, 2);
        else SGL_SPLIT(128, PREFIX_DEPTH, 4);
    } else {
        if (wpg == 1) { if (a.kind == 1) SGL_SPLIT(64, PREFIX_DEPTH, 1); else SGL_SPLIT(64, 1, 1); }
        else SGL_SPLIT(64, PREFIX_DEPTH, 2);
    }
#undef SGL_SPLIT
    return hip_status(hipGetLastError());
}

int launch_split_fp8(const SplitArgs &a0, hipStream_t st) {
    if (a0.kind == 4) return SGL_ERR_UNSUPPORTED;   // small-q extend runs on bf16 caches only
    if ((a0.n_sets == 0 || a0.max_splits == 0) && a0.store.n_tokens == 0 && !a0.store.ss.lo) return SGL_OK;
    if (a0.chunk % TILE8 != 0 || !a0.k_scale || !a0.v_scale) return SGL_ERR_INVALID;
    SplitArgs a = a0;
    const int rows = (a.kind == 1 ? a.max_members : 1) * (a.Hq / a.Hkv);
    a.row_blocks = (rows + 15) / 16;
    // same work split as launch_split_bf16
    int wpg = 1;
    if (a.kind == 1) wpg = a.row_blocks >= 3 ? 4 : a.row_blocks;
    if (a.D == 64 && wpg > 2) wpg = 2;               // 2 load instructions per 64-dim tile
    const int n_rbg = (a.row_blocks + wpg - 1) / wpg;
    const int64_t items = (int64_t)a.n_sets * a.max_splits * a.Hkv;
    int rc = carried_store(a, true, 64 * wpg);
    if (rc != SGL_OK) return rc;
    const int64_t n_wg = ceil_div64(items, 8) * 8 * n_rbg + a.store.n_wg;
    if (n_wg > 0x7fffffff) return SGL_ERR_UNSUPPORTED;
    const size_t dyn = (size_t)a.chunk * sizeof(int32_t);
    const dim3 grid((unsigned)n_wg), block(64 * wpg);
#define SGL_SPLIT8(DD, DP, W) hipLaunchKernelGGL((split_fp8_kernel<DD, DP, W>), grid, block, dyn, st, a)
    if (a.D == 128) {
        if (wpg == 1) { if (a.kind == 1) SGL_SPLIT8(128, PREFIX_DEPTH, 1); else SGL_SPLIT8(128, 1, 1); }
        else if (wpg == 2) SGL_SPLIT8(128, PREFIX_DEPTH, 2);
        else SGL_SPLIT8(128, PREFIX_DEPTH, 4);
    } else {
        if (wpg == 1) { if (a.kind == 1) SGL_SPLIT8(64, PREFIX_DEPTH, 1); else SGL_SPLIT8(64, 1, 1); }
        else SGL_SPLIT8(64, PREFIX_DEPTH, 2);
    }
#undef SGL_SPLIT8
    return hip_status(hipGetLastError());
}
