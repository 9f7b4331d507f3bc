// kernels_misc.hip -- req_to_token build, KV store, and the log-sum-exp merge
// of partial softmax states.
#include <cstring>

#include "store_util.h"

// ---------------------------------------------------------------------------
// req_to_token build: one workgroup per request, columns strided over threads.
// Row r of the batch writes table row req_rows[r]: columns [0, P_r) from the
// prefix CSR and [c0, c0 + E_r) from the new-slot CSR ("SGLang 深度解读"
// module 5: req_to_token maps a request's token positions to pool slots).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) r2t_build_kernel(
    int32_t *__restrict__ r2t, int64_t num_rows, int64_t stride, const int32_t *__restrict__ req_rows,
    int32_t batch, const int32_t *__restrict__ prefix_slots, const int64_t *__restrict__ prefix_off,
    const int32_t *__restrict__ new_slots, const int64_t *__restrict__ new_off,
    const int32_t *__restrict__ new_col0) {
    const int r = blockIdx.x;
    const int64_t row = req_rows[r];
    if (row < 0 || row >= num_rows) return;
    int32_t *dst = r2t + row * stride;
    int64_t P = 0;
    if (prefix_off) {
        const int64_t a = prefix_off[r], b = prefix_off[r + 1], total = prefix_off[batch];
        if (a >= 0 && a <= b && b <= total) {
            P = b - a;
            for (int64_t j = threadIdx.x; j < P && j < stride; j += blockDim.x) dst[j] = prefix_slots[a + j];
        }
    }
    const int64_t a = new_off[r], b = new_off[r + 1], total = new_off[batch];
    if (!(a >= 0 && a <= b && b <= total)) return;
    const int64_t c0 = new_col0 ? (int64_t)new_col0[r] : P;
    for (int64_t j = threadIdx.x; j < b - a; j += blockDim.x) {
        const int64_t c = c0 + j;
        if (c >= 0 && c < stride) dst[c] = new_slots[a + j];
    }
}

int launch_build_req_to_token(int32_t *r2t, int64_t num_rows, int64_t row_stride,
                              const int32_t *req_rows, int32_t batch, const int32_t *prefix_slots,
                              const int64_t *prefix_off, const int32_t *new_slots,
                              const int64_t *new_off, const int32_t *new_col0, hipStream_t st) {
    if (batch == 0) return SGL_OK;
    hipLaunchKernelGGL(r2t_build_kernel, dim3(batch), dim3(256), 0, st, r2t, num_rows, row_stride,
                       req_rows, batch, prefix_slots, prefix_off, new_slots, new_off, new_col0);
    return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Index check on the device: count the slot ids of the requests' rows that lie
// outside the pool (the attention kernels read slot 0 in their place), and
// the requests whose row or length is out of range.  Grid (key chunks,
// batch); a wave counts its 64 ids by ballot and adds the count with one
// vector atomic.
// ---------------------------------------------------------------------------
constexpr int kCheckChunk = 4096;   // keys per workgroup

__global__ void __launch_bounds__(256) count_bad_slots_kernel(
    const int32_t *__restrict__ r2t, int64_t num_rows, int64_t stride, const int32_t *__restrict__ req_rows,
    const int32_t *__restrict__ seq_lens, int64_t max_len, int64_t num_slots, uint32_t *__restrict__ count) {
    const int r = blockIdx.y;
    const int64_t row = req_rows[r];
    const int64_t L = seq_lens[r];
    const int lane = threadIdx.x & 63;
    if (row < 0 || row >= num_rows || L < 0 || L > stride || L > max_len) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(count, 1u);
        return;
    }
    const int32_t *src = r2t + row * stride;
    const int64_t k0 = (int64_t)blockIdx.x * kCheckChunk;
    const int64_t k1 = k0 + kCheckChunk < L ? k0 + kCheckChunk : L;
    uint32_t bad = 0;
    for (int64_t j = k0 + threadIdx.x; j - threadIdx.x < k1; j += blockDim.x) {
        const bool out = j < k1 && (src[j] < 0 || (int64_t)src[j] >= num_slots);
        bad += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(out));
    }
    if (lane == 0 && bad) atomicAdd(count, bad);
}

int launch_count_bad_slots(const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                           uint32_t *count, hipStream_t st) {
    if (batch == 0) return SGL_OK;
    const int64_t chunks = max_seq_len > 0 ? ceil_div64(max_seq_len, kCheckChunk) : 1;
    if (chunks > 65535 || batch > 65535) return SGL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(count_bad_slots_kernel, dim3((unsigned)chunks, (unsigned)batch), dim3(256), 0, st, r2t,
                       num_rows, row_stride, req_rows, seq_lens, (int64_t)max_seq_len, num_slots, count);
    return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------------------
// KV store: copy token rows (Hkv * D elements = row_chunks * 16 bytes) of K and
// V into the pools at their slots ("SGLang 深度解读" module 5: write the
// current K, V at cache_loc before attending).  Modes 0 (given slots) and 1
// (extend: the slots of positions prefix_lens[r] + i) here; mode 2 (decode)
// is decode_store_job (store_util.h), which a cascade call may instead hand
// to the leading workgroups of its prefix-stage launch.
// ---------------------------------------------------------------------------
// The suffix starts; with a.plan the last workgroup computes the balanced
// suffix stage's plan instead.
__global__ void __launch_bounds__(256) suffix_start_kernel(SuffixStartArgs a) {
    const unsigned n = gridDim.x - (a.plan ? 1u : 0u);
    if (blockIdx.x >= n) {
        balanced_plan(a);
        return;
    }
    suffix_starts(a, blockIdx.x, n);
}

int launch_suffix_start(const SuffixStartArgs &a, hipStream_t st) {
    if (a.batch <= 0) return SGL_OK;
    if (a.G < 1 || !a.lo || (a.plan && a.plan_wgs < 1)) return SGL_ERR_INVALID;
    const unsigned n = (unsigned)ceil_div64(a.batch, 256) + (a.plan ? 1u : 0u);
    hipLaunchKernelGGL(suffix_start_kernel, dim3(n), dim3(256), 0, st, a);
    return hip_status(hipGetLastError());
}

template <int MODE>
__global__ void __launch_bounds__(256) store_kv_kernel(
    const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new, uint4 *__restrict__ k_pool,
    uint4 *__restrict__ v_pool, int64_t num_slots, int32_t row_chunks, int64_t n_tokens,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ r2t, int64_t num_rows,
    int64_t stride, const int32_t *__restrict__ req_rows, const int32_t *__restrict__ lens,
    const int64_t *__restrict__ q_off) {
    if (MODE == 1) {
        // extend: blockIdx.y = request; tokens q_off[r] .. q_off[r+1]
        const int r = blockIdx.y;
        const int64_t t0 = q_off[r], t1 = q_off[r + 1];
        const int64_t row = req_rows[r];
        const int64_t P = lens[r];
        if (row < 0 || row >= num_rows || t0 < 0 || t1 > n_tokens || t0 > t1 || P < 0) return;
        const int64_t n = (t1 - t0) * row_chunks;
        for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
             idx += (int64_t)gridDim.x * blockDim.x) {
            const int64_t i = idx / row_chunks, c = idx % row_chunks;
            const int64_t col = P + i;
            if (col >= stride) continue;
            const int32_t s = r2t[row * stride + col];
            if (s < 0 || s >= num_slots) continue;
            k_pool[(int64_t)s * row_chunks + c] = k_new[(t0 + i) * row_chunks + c];
            v_pool[(int64_t)s * row_chunks + c] = v_new[(t0 + i) * row_chunks + c];
        }
    } else {
        const int64_t n = n_tokens * row_chunks;
        for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
             idx += (int64_t)gridDim.x * blockDim.x) {
            const int64_t i = idx / row_chunks, c = idx % row_chunks;
            const int32_t s = slots[i];
            if (s < 0 || s >= num_slots) continue;
            k_pool[(int64_t)s * row_chunks + c] = k_new[i * row_chunks + c];
            v_pool[(int64_t)s * row_chunks + c] = v_new[i * row_chunks + c];
        }
    }
}

template <int ELT, bool FP8>
__global__ void __launch_bounds__(256) decode_store_kernel(DecodeStoreArgs d) {
    const unsigned n = gridDim.x - (d.ss.plan ? 1u : 0u);   // the last workgroup: the plan (launch_decode_store)
    if (blockIdx.x >= n) {
        balanced_plan(d.ss);
        return;
    }
    decode_store_job<ELT, FP8>(d, blockIdx.x, n);
}

DecodeStoreArgs decode_store_args(int elt, bool fp8, const void *k_new, const void *v_new, int64_t n_tokens,
                                  void *k_pool, void *v_pool, int64_t num_slots, int32_t Hkv, int32_t D,
                                  const float *k_scale, const float *v_scale, const int32_t *r2t,
                                  int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                                  const int32_t *lens, const SuffixStartArgs *ss) {
    DecodeStoreArgs d;
    std::memset(&d, 0, sizeof d);
    d.k_new = (const char *)k_new; d.v_new = (const char *)v_new;
    d.k_pool = (uint4 *)k_pool; d.v_pool = (uint4 *)v_pool;
    d.num_slots = num_slots;
    d.row_chunks = fp8 ? Hkv * D / 16 : (int32_t)((int64_t)Hkv * D * elt / 16);
    d.head_chunks = D / 16;
    d.k_scale = k_scale; d.v_scale = v_scale;
    d.r2t = r2t; d.num_rows = num_rows; d.stride = row_stride;
    d.req_rows = req_rows; d.lens = lens;
    d.n_tokens = k_new ? n_tokens : 0;
    d.elt = elt; d.fp8 = fp8 ? 1 : 0;
    if (ss) d.ss = *ss;
    return d;
}

int32_t decode_store_wgs(const DecodeStoreArgs &d, int threads) {
    const int64_t chunks = d.n_tokens * d.row_chunks;
    const int64_t starts = d.ss.lo ? d.ss.batch : 0;
    if (chunks <= 0 && starts <= 0) return 0;
    // about four chunks per thread, and (decode_store_job) as many more
    // workgroups for the suffix starts
    int64_t n = ceil_div64(chunks, 4 * (int64_t)threads) + ceil_div64(starts, threads);
    n = std::min<int64_t>(std::max<int64_t>(n, 1), 256);
    return (int32_t)ceil_div64(n, 8) * 8;
}

// the decode store (and suffix starts) in a launch of its own
static int launch_decode_store(const DecodeStoreArgs &d, hipStream_t st) {
    if (d.n_tokens == 0) return SGL_OK;
    if (d.fp8 && (!d.k_scale || !d.v_scale)) return SGL_ERR_INVALID;
    const int64_t store_wgs = std::min<int64_t>(ceil_div64(d.n_tokens * d.row_chunks, 256), 8192);
    if (d.ss.plan && (!d.ss.lo || d.ss.plan_wgs < 1)) return SGL_ERR_INVALID;
    const dim3 grid((unsigned)(store_wgs + (d.ss.lo ? ceil_div64(d.ss.batch, 256) : 0) + (d.ss.plan ? 1 : 0)));
    if (!d.fp8) hipLaunchKernelGGL((decode_store_kernel<2, false>), grid, dim3(256), 0, st, d);
    else if (d.elt == 2) hipLaunchKernelGGL((decode_store_kernel<2, true>), grid, dim3(256), 0, st, d);
    else hipLaunchKernelGGL((decode_store_kernel<4, true>), grid, dim3(256), 0, st, d);
    return hip_status(hipGetLastError());
}

int launch_store_kv(int mode, int elt, const void *k_new, const void *v_new, int64_t n_tokens,
                    const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                    int32_t Hkv, int32_t D, const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                    const int32_t *req_rows, const int32_t *lens, const int64_t *q_off,
                    int32_t batch, int32_t max_extend_len, hipStream_t st, const SuffixStartArgs *ss) {
    if (n_tokens == 0) return SGL_OK;
    if (mode == 2)
        return launch_decode_store(decode_store_args(elt, false, k_new, v_new, n_tokens, k_pool, v_pool, num_slots,
                                                     Hkv, D, nullptr, nullptr, r2t, num_rows, row_stride,
                                                     req_rows, lens, ss),
                                   st);
    const int32_t row_chunks = (int32_t)((int64_t)Hkv * D * elt / 16);
    const uint4 *kn = (const uint4 *)k_new;
    const uint4 *vn = (const uint4 *)v_new;
    uint4 *kp = (uint4 *)k_pool;
    uint4 *vp = (uint4 *)v_pool;
    if (mode == 1) {
        int64_t per_req = (int64_t)max_extend_len * row_chunks;
        int gx = (int)std::min<int64_t>(ceil_div64(per_req, 256), 1024);
        if (gx < 1) gx = 1;
        hipLaunchKernelGGL(store_kv_kernel<1>, dim3(gx, batch), dim3(256), 0, st, kn, vn, kp, vp,
                           num_slots, row_chunks, n_tokens, slots, r2t, num_rows, row_stride,
                           req_rows, lens, q_off);
    } else {
        int gx = (int)std::min<int64_t>(ceil_div64(n_tokens * row_chunks, 256), 8192);
        hipLaunchKernelGGL(store_kv_kernel<0>, dim3(gx), dim3(256), 0, st, kn, vn, kp, vp,
                           num_slots, row_chunks, n_tokens, slots, r2t, num_rows, row_stride,
                           req_rows, lens, q_off);
    }
    return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------------------
// FP8 KV store: the same rows as store_kv_kernel, quantised to e4m3fn codes on
// the way by quant16 (store_util.h).  One thread writes one 16-byte chunk of
// codes.
// ---------------------------------------------------------------------------
template <int MODE, int ELT>
__global__ void __launch_bounds__(256) store_kv_fp8_kernel(
    const char *__restrict__ k_new, const char *__restrict__ v_new, uint4 *__restrict__ k_pool,
    uint4 *__restrict__ v_pool, int64_t num_slots, int32_t row_chunks, int32_t head_chunks,
    const float *__restrict__ k_scale, const float *__restrict__ v_scale, int64_t n_tokens,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ r2t, int64_t num_rows,
    int64_t stride, const int32_t *__restrict__ req_rows, const int32_t *__restrict__ lens,
    const int64_t *__restrict__ q_off) {
    constexpr int IN_CHUNK = 16 * ELT;   // input bytes per 16 codes
    int64_t t0 = 0, n = n_tokens * row_chunks, row = 0, P = 0;
    if (MODE == 1) {
        const int r = blockIdx.y;
        t0 = q_off[r];
        const int64_t t1 = q_off[r + 1];
        row = req_rows[r];
        P = lens[r];
        if (row < 0 || row >= num_rows || t0 < 0 || t1 > n_tokens || t0 > t1 || P < 0) return;
        n = (t1 - t0) * row_chunks;
    }
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / row_chunks, c = idx % row_chunks;
        int32_t s;
        if (MODE == 0) {
            s = slots[i];
        } else {
            const int64_t col = P + i;
            if (col >= stride) continue;
            s = r2t[row * stride + col];
        }
        if (s < 0 || s >= num_slots) continue;
        const int h = (int)(c / head_chunks);
        const int64_t src = ((t0 + i) * row_chunks + c) * IN_CHUNK;
        k_pool[(int64_t)s * row_chunks + c] = quant16<ELT>(k_new + src, k_scale[h]);
        v_pool[(int64_t)s * row_chunks + c] = quant16<ELT>(v_new + src, v_scale[h]);
    }
}

int launch_store_kv_fp8(int mode, int elt, const void *k_new, const void *v_new, int64_t n_tokens,
                        const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                        int32_t Hkv, int32_t D, const float *k_scale, const float *v_scale,
                        const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                        const int32_t *req_rows, const int32_t *lens, const int64_t *q_off,
                        int32_t batch, int32_t max_extend_len, hipStream_t st, const SuffixStartArgs *ss) {
    if (n_tokens == 0) return SGL_OK;
    if (mode == 2)
        return launch_decode_store(decode_store_args(elt, true, k_new, v_new, n_tokens, k_pool, v_pool, num_slots,
                                                     Hkv, D, k_scale, v_scale, r2t, num_rows, row_stride,
                                                     req_rows, lens, ss),
                                   st);
    const int32_t row_chunks = Hkv * D / 16, head_chunks = D / 16;
    const char *kn = (const char *)k_new;
    const char *vn = (const char *)v_new;
    uint4 *kp = (uint4 *)k_pool;
    uint4 *vp = (uint4 *)v_pool;
    dim3 grid;
    if (mode == 1) {
        const int64_t per_req = (int64_t)max_extend_len * row_chunks;
        const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div64(per_req, 256), 1024));
        grid = dim3(gx, batch);
    } else {
        grid = dim3((unsigned)std::min<int64_t>(ceil_div64(n_tokens * row_chunks, 256), 8192));
    }
#define SGL_STORE8(M, E)                                                                                    \
    hipLaunchKernelGGL((store_kv_fp8_kernel<M, E>), grid, dim3(256), 0, st, kn, vn, kp, vp, num_slots,     \
                       row_chunks, head_chunks, k_scale, v_scale, n_tokens, slots, r2t, num_rows,          \
                       row_stride, req_rows, lens, q_off)
    if (elt == 2) {
        if (mode == 0) SGL_STORE8(0, 2); else SGL_STORE8(1, 2);
    } else {
        if (mode == 0) SGL_STORE8(0, 4); else SGL_STORE8(1, 4);
    }
#undef SGL_STORE8
    return hip_status(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Merge of partial softmax states.  The pages give the one-key online-softmax
// update (rescale what was accumulated by e^(m_old - m_new), chenxutan.com
// section 3.2 PagedPrefill); applied to whole blocks it is
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s o_s 2^(m_s - M) / L
// (m in log2 units).  One wave per (request, q head); lanes own dims.
// ---------------------------------------------------------------------------

template <int D, bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)a.batch * a.Hq) return;
    const int r = (int)(item / a.Hq), h = (int)(item % a.Hq);

    // parts: [prefix splits of r][suffix (or flat) splits of r]
    int np = 0, ns;
    int64_t sk_w0 = 0;      // balanced suffix stage: the first run covering r
    if (a.kind == 4 || a.kind == 5) {
        // token r of request rq = the last rq with q_off[rq] <= r
        int lo = 0, hi = a.n_req - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.q_off[mid] <= r) lo = mid; else hi = mid - 1;
        }
        const int64_t P = a.prefix_lens[lo], E = a.q_off[lo + 1] - a.q_off[lo];
        if (a.kind == 4) {
            const int64_t L = (P < 0 ? 0 : P) + E;
            ns = L > 0 ? (int)ceil_div64(L, verify_chunk(L, a.n_spl)) : 0;
        } else {
            // the keys of the query tile holding token i of the request: as the
            // prefill kernel bounds them (128 query rows per tile)
            const int64_t tpt = kExtendTileRows / (a.Hq / a.Hkv);
            const int64_t i = r - a.q_off[lo];
            const int64_t q0 = i / tpt * tpt;
            int64_t kv_end = (P < 0 ? 0 : P) + (q0 + tpt < E ? q0 + tpt : E);
            if (kv_end > a.row_stride) kv_end = a.row_stride;
            ns = kv_end > 0 ? (int)ceil_div64(kv_end, a.chunk_flat) : 0;
        }
    } else {
        const int64_t L = a.seq_lens[r];
        if (a.kind == 3) {
            int64_t P = a.suffix_lo ? a.suffix_lo[r] : a.group_prefix_len[wave_find_group(a.group_ptr, a.G, r)];
            P = P < 0 ? 0 : (P > L ? L : P);
            np = (int)ceil_div64(P, a.chunk_prefix);
            if (a.sk_plan) {
                // balanced suffix stage: the pieces of r are rows r + w of
                // the runs w that cover its suffix keys
                const int64_t off = a.sk_plan[r], nxt = a.sk_plan[r + 1], C = a.sk_plan[a.batch + 1];
                sk_w0 = nxt > off ? off / C : 0;
                ns = nxt > off ? (int)((nxt - 1) / C - sk_w0 + 1) : 0;
            } else {
                ns = (int)ceil_div64(L - P, a.chunk_flat);
            }
        } else {
            ns = (int)ceil_div64(L, a.chunk_flat);
        }
    }
    if (np > a.prefix.S) np = a.prefix.S;
    const bool sk = a.kind == 3 && a.sk_plan;
    if (!sk && ns > a.flat_or_suffix.S) ns = a.flat_or_suffix.S;
    const int total = np + ns;

    // state row of part s
    auto row_of = [&](int s) -> int64_t {
        if (s < np) return (int64_t)r * a.prefix.S + s;
        return sk ? r + sk_w0 + (s - np) : (int64_t)r * a.flat_or_suffix.S + (s - np);
    };
    auto ml_of = [&](int s) -> float2 {
        const PartialBuf &pb = s < np ? a.prefix : a.flat_or_suffix;
        const float *p = pb.ml + (row_of(s) * a.Hq + h) * 2;
        return make_float2(p[0], p[1]);
    };
    auto o_of = [&](int s) -> const float * {
        const PartialBuf &pb = s < np ? a.prefix : a.flat_or_suffix;
        return pb.o + (row_of(s) * a.Hq + h) * D;
    };

    constexpr int PER = D / 64;
    const int64_t obase = ((int64_t)r * a.Hq + h) * D + lane * PER;
    // Up to FAST parts (head dims up to 128): every part's (m, l) -- lane j
    // holds part j's -- and o row are loaded at once, so the merge waits for
    // one round of loads instead of one per pass over the states.  16 parts
    // cover the decode and cascade splits of contexts up to 8k keys; 32
    // measured slower (their 64 o registers cost the kernel occupancy: 11.7
    // against 9.0 us per merge on the 256-request decode workload).
    constexpr int FAST = PER <= 2 ? 16 : 0;
    if (FAST > 0 && total <= FAST) {
        float2 v = make_float2(-INFINITY, 0.f);
        if (lane < total) v = ml_of(lane);
        float ov[FAST > 0 ? FAST : 1][PER];
#pragma unroll
        for (int u = 0; u < FAST; u++) {
            if (u < total) {
                const float *op = o_of(u);
#pragma unroll
                for (int i = 0; i < PER; i++) ov[u][i] = op[lane * PER + i];
            } else {
#pragma unroll
                for (int i = 0; i < PER; i++) ov[u][i] = 0.f;
            }
        }
        const float M = wave_max(v.y > 0.f ? v.x : -INFINITY);
        const float f = v.y > 0.f ? exp2f(v.x - M) : 0.f;
        const float Lsum = wave_sum(v.y > 0.f ? v.y * f : 0.f);
        float acc[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) acc[i] = 0.f;
#pragma unroll
        for (int u = 0; u < FAST; u++) {
            const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u));
#pragma unroll
            for (int i = 0; i < PER; i++) acc[i] += fu == 0.f ? 0.f : ov[u][i] * fu;
        }
        const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            if (OUT_BF16)
                ((__bf16 *)a.o)[obase + i] = (__bf16)(acc[i] * inv);
            else
                ((float *)a.o)[obase + i] = acc[i] * inv;
        }
        if (a.lse && lane == 0)
            a.lse[(int64_t)r * a.Hq + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
        return;
    }

    // lane j holds the state of parts j, j + 64, ...: the maximum first, then
    // each part's weight 2^(m - M) (0 for an empty part), broadcast by
    // readlane while the o rows of eight parts are in flight at once
    float M = -INFINITY;
    for (int s0 = 0; s0 < total; s0 += 64) {
        const int s = s0 + lane;
        float m = -INFINITY;
        if (s < total) {
            float2 v = ml_of(s);
            if (v.y > 0.f) m = v.x;
        }
        M = fmaxf(M, wave_max(m));
    }
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) acc[i] = 0.f;
    float Lpart = 0.f;
    for (int s0 = 0; s0 < total; s0 += 64) {
        const int s = s0 + lane;
        float f = 0.f;
        if (s < total) {
            const float2 v = ml_of(s);
            if (v.y > 0.f) {
                f = exp2f(v.x - M);
                Lpart += v.y * f;
            }
        }
        const int cnt = total - s0 < 64 ? total - s0 : 64;
        for (int u0 = 0; u0 < cnt; u0 += 8) {
            float ov[8][PER], fu[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int uu = u0 + u < cnt ? u0 + u : cnt - 1;
                fu[u] = u0 + u < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), uu)) : 0.f;
                const float *op = o_of(s0 + uu);
#pragma unroll
                for (int i = 0; i < PER; i++) ov[u][i] = op[lane * PER + i];
            }
#pragma unroll
            for (int u = 0; u < 8; u++)
#pragma unroll
                for (int i = 0; i < PER; i++) acc[i] += fu[u] == 0.f ? 0.f : ov[u][i] * fu[u];
        }
    }
    const float Lsum = wave_sum(Lpart);
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        if (OUT_BF16)
            ((__bf16 *)a.o)[obase + i] = (__bf16)(acc[i] * inv);
        else
            ((float *)a.o)[obase + i] = acc[i] * inv;
    }
    if (a.lse && lane == 0)
        a.lse[(int64_t)r * a.Hq + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

int launch_merge(const MergeArgs &a, hipStream_t st) {
    const int64_t items = (int64_t)a.batch * a.Hq;
    if (items == 0) return SGL_OK;
    dim3 grid((unsigned)ceil_div64(items, 4)), block(256);
    if (a.D == 512) {   // latent (MLA) values, bf16 only
        if (!a.out_bf16) return SGL_ERR_UNSUPPORTED;
        hipLaunchKernelGGL((merge_kernel<512, true>), grid, block, 0, st, a);
    } else if (a.D == 128) {
        if (a.out_bf16) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, st, a);
    } else {
        if (a.out_bf16) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, st, a);
    }
    return hip_status(hipGetLastError());
}
