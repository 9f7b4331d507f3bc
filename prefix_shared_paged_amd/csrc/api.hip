// api.hip -- C-ABI device entry points of libsgl_attn: argument checks,
// optional host-side validation of index metadata, workspace layout, and the
// kernel launches.  See include/sgl_attn.h for the contract.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"

namespace {

constexpr int kDecodeChunk = 1024;   // keys per split of the per-head kernels (flat, suffix)
constexpr int kRowsChunk = 512;      // keys per split of the whole-row kernel (flat fp8)
constexpr int kSuffixChunk = 1024;   // keys per split of the cascade suffix (whole-row kernel), at most
constexpr int kPrefixChunkMax = 512;
constexpr int kPrefixChunkMin = 128;
constexpr int64_t kPrefixWorkgroups = 1024;  // ~4 per compute unit
constexpr int kFlatXcdBlock = 16;    // consecutive requests per XCD block (flat fp8 decode)
constexpr size_t kAlign = 256;
// Split-state scratch of the allocation-free cascade decode (per GPU).
constexpr size_t kStaticScratchBytes = size_t(128) << 20;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Keys per split of the cascade prefix stage.  The stage runs one workgroup
// per (group, KV head, split, block of up to 4 x 16 query rows) -- often far
// fewer than the flat call has work items -- and a workgroup walks its
// split's tiles one after another, so the splits are halved (down to
// kPrefixChunkMin keys) until about kPrefixWorkgroups workgroups run.  The
// row-block rule matches the launcher in kernels_decode.hip.  Splits shorter
// than 128 keys cost more in per-workgroup start-up (slot table, queries,
// state writes) than their parallelism gains: the extend step's decode (64
// requests over one 2,048-key prefix, 257-key suffixes) takes 40 us with
// 128-key prefix and suffix splits against 50 us with 64 and 44 us with 256.
int prefix_chunk(int32_t G, int32_t max_group_size, int32_t max_prefix_len, int32_t Hq, int32_t Hkv, int32_t D) {
    const int64_t rb = ceil_div64((int64_t)max_group_size * (Hq / Hkv), 16);
    int64_t wpg = rb >= 3 ? 4 : rb;
    if (D == 64 && wpg > 2) wpg = 2;
    const int64_t units = (int64_t)G * Hkv * ceil_div64(rb, wpg);
    int c = kPrefixChunkMax;
    while (c > kPrefixChunkMin && units * ceil_div64(max_prefix_len, c) < kPrefixWorkgroups) c /= 2;
    return c;
}

// Keys per split of the cascade suffix stage (the whole-row kernel, one
// workgroup per (request, 4 KV heads, split)).  kSuffixChunk normally: on the
// 256-request decode workload 1024-key splits take 641 us against 653 us with
// 512 (each workgroup hand-off on a compute unit -- draining the finished
// item's state stores, starting the next -- leaves its slot idle for a few
// us, and the prefix items that follow the suffix rounds fill the longer
// tail).  Halved (down to kPrefixChunkMin) while the suffixes -- estimated as
// max_seq_len - max_prefix_len, which only sizes the splits -- would give
// fewer than kPrefixWorkgroups workgroups: a batch of a few dozen requests
// with short suffixes otherwise leaves most compute units idle while each
// workgroup walks its suffix alone.
int suffix_chunk(int32_t batch, int32_t max_seq_len, int32_t max_prefix_len, int32_t Hkv) {
    const int64_t units = (int64_t)batch * (Hkv > 4 ? Hkv / 4 : 1);
    const int64_t est = std::max<int64_t>(1, (int64_t)max_seq_len - std::max<int32_t>(max_prefix_len, 0));
    int c = kSuffixChunk;
    while (c > kPrefixChunkMin && units * ceil_div64(est, c) < kPrefixWorkgroups) c /= 2;
    return c;
}

// Validation mode: -1 follows the SGL_ATTN_VALIDATE environment variable
// (read once), 0 / 1 are set by sgl_set_validate.
std::atomic<int> g_validate_mode{-1};

bool validate_on() {
    const int m = g_validate_mode.load(std::memory_order_relaxed);
    if (m >= 0) return m == 1;
    static const bool env = [] {
        const char *e = std::getenv("SGL_ATTN_VALIDATE");
        return e && e[0] && e[0] != '0';
    }();
    return env;
}

bool shape_ok(int dtype, int32_t Hq, int32_t Hkv, int32_t D) {
    if (dtype != SGL_F32 && dtype != SGL_BF16) return false;
    if (D != 64 && D != 128) return false;
    if (Hkv < 1 || Hkv > 16 || Hq < Hkv || Hq % Hkv != 0) return false;
    const int g = Hq / Hkv;
    return g == 1 || g == 2 || g == 4 || g == 8;
}

int elt_size(int dtype) { return dtype == SGL_BF16 ? 2 : 4; }

template <class T>
bool fetch(std::vector<T> &out, const T *dev, size_t n, hipStream_t st) {
    out.resize(n);
    if (n == 0) return true;
    if (hipStreamSynchronize(st) != hipSuccess) return false;
    return hipMemcpy(out.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

size_t part_bytes(int64_t B, int64_t S, int64_t Hq, int64_t D) {
    return align_up((size_t)(B * S * Hq * D) * sizeof(float)) + align_up((size_t)(B * S * Hq * 2) * sizeof(float));
}

// Workgroups per head group of the balanced suffix stage: four per compute
// unit over the whole grid.
constexpr int kBalancedWorkgroups = 1024;
int64_t balanced_wgs(int32_t Hkv) { return kBalancedWorkgroups / (Hkv >= 4 ? Hkv / 4 : 1); }

// Bytes of the cascade's suffix states: Ss splits per request, or the rows
// of the balanced suffix stage, whichever is larger (one region serves both).
size_t suffix_part_bytes(int64_t B, int64_t Ss, int64_t Hq, int64_t Hkv, int64_t D) {
    return std::max(part_bytes(B, Ss, Hq, D), part_bytes(sk_state_rows(B, balanced_wgs((int32_t)Hkv)), 1, Hq, D));
}

PartialBuf carve(char *&p, int64_t B, int64_t S, int64_t Hq, int64_t D) {
    PartialBuf pb;
    pb.o = (float *)p;
    p += align_up((size_t)(B * S * Hq * D) * sizeof(float));
    pb.ml = (float *)p;
    p += align_up((size_t)(B * S * Hq * 2) * sizeof(float));
    pb.S = (int32_t)S;
    return pb;
}

// Check that req_to_token row `row` columns [c0, c1) hold valid slots.
bool slots_ok(const std::vector<int32_t> &tab, int64_t row_stride, int64_t row, int64_t c0, int64_t c1,
              int64_t num_slots) {
    for (int64_t c = c0; c < c1; c++) {
        const int32_t s = tab[(size_t)(row * row_stride + c)];
        if (s < 0 || s >= num_slots) return false;
    }
    return true;
}

// Small-q extend (a few new tokens per request over a long cached context,
// the verify step of speculative decoding): when every request's new tokens
// times the query heads per KV head fit one 16-row MFMA block, the extend
// runs as a split-K decode of those rows -- each request's keys cut into
// n_spl splits, one wave per (request, KV head, split) -- and a log-sum-exp
// merge, instead of the 128-row tiles of the prefill kernel, which stream
// each long context through one workgroup per KV head with most rows empty.
// Measured on 64 requests over contexts of 2-8k keys (32/8 heads): 1, 2, 4
// new tokens take 287, 293, 310 us this way against 336, 332, 326 us in the
// prefill kernel; with 32 or 64 rows per KV head (several waves sharing each
// tile) the split-K form is slower, so those stay in the prefill kernel.
constexpr int kSmallQRows = 16;
bool small_q_extend(int32_t max_extend_len, int32_t Hq, int32_t Hkv) {
    return Hkv > 0 && (int64_t)max_extend_len * (Hq / Hkv) <= kSmallQRows;
}
// Key splits of the prefill kernel.  Its grid has one workgroup per
// (request, tile of 128 query rows, KV head), each walking all of its keys;
// when that grid has at most one workgroup per compute unit (one or two long
// requests, as in the last rounds of chunked prefill) and rows may be long,
// each workgroup's keys are cut into splits of ksplit keys (a multiple of
// 4096, so a split starts where the kernel's slot table starts a fill) so
// that about kExtendWgTarget workgroups run; row_stride bounds every context.
// Measured on 64/8 heads with the two-waves-per-SIMD kernel: one request over
// 30k keys (128 workgroups) 554 -> 328 us, over 20k keys (256) 451 -> 425 us;
// with 512 or more workgroups the splits' merge costs more than it gains, so
// they run unsplit.
constexpr int64_t kExtendSplitKeys = 4096;
constexpr int64_t kExtendWgTarget = 1024;
constexpr int64_t kExtendSplitMaxWg = 256;
int32_t extend_key_splits(int32_t batch, int32_t max_extend_len, int64_t row_stride, int32_t Hq, int32_t Hkv,
                          int32_t *ksplit) {
    const int64_t g = Hq / Hkv;
    const int64_t n_wg = ceil_div64(max_extend_len, kExtendTileRows / g) * batch * Hkv;
    const int64_t chunks = ceil_div64(row_stride, kExtendSplitKeys);
    int64_t S = 1;
    if (n_wg <= kExtendSplitMaxWg && chunks >= 2) S = std::min(chunks, ceil_div64(kExtendWgTarget, n_wg));
    const int64_t per = ceil_div64(chunks, S);
    *ksplit = (int32_t)(per * kExtendSplitKeys);
    return (int32_t)ceil_div64(row_stride, per * kExtendSplitKeys);
}

int32_t extend_splits(int32_t batch, int32_t Hkv) {
    const int64_t items = (int64_t)batch * Hkv;
    int64_t n = items > 0 ? (2048 + items - 1) / items : 1;
    return (int32_t)(n < 1 ? 1 : (n > 8 ? 8 : n));
}

// MLA latent decode: keys per split of the flat call and the suffix, and
// the prefix split (halved down to kPrefixChunkMin keys until about kPrefixWorkgroups
// workgroups run; the row-block rule matches launch_split_mla).
// Keys per flat / suffix split of the latent decode: 512 below 64 query rows
// per split; from 64 rows on the split states (512 fp32 per row and split)
// would otherwise cost as much traffic as the latents, so 2048 at exactly 64
// rows (one workgroup per split; 258 -> 244 us on the latent workload) and
// 1024 above, where two or more workgroups share each split and the grid
// would be too small with 2048 (398 -> 421 us at 128 heads).
int mla_chunk(int32_t Hq) { return Hq > 64 ? 1024 : (Hq == 64 ? 2048 : 512); }
constexpr int kMlaDqk = 576, kMlaDv = 512;
int mla_prefix_chunk(int32_t G, int32_t max_group_size, int32_t max_prefix_len, int32_t Hq) {
    const int64_t rb = ceil_div64((int64_t)max_group_size * Hq, 16);
    const int64_t rbw = rb >= 4 ? 4 : (rb >= 2 ? 2 : 1);
    const int64_t units = (int64_t)G * ceil_div64(rb, rbw);
    int c = kPrefixChunkMax;
    while (c > kPrefixChunkMin && units * ceil_div64(max_prefix_len, c) < kPrefixWorkgroups) c /= 2;
    return c;
}

}  // namespace

extern "C" {

int sgl_abi_version(void) { return 5; }

int sgl_set_validate(int mode) {
    if (mode < -1 || mode > 1) return -2;
    return g_validate_mode.exchange(mode);
}

int sgl_build_req_to_token(int32_t *r2t, int64_t num_rows, int64_t row_stride,
                           const int32_t *req_rows, int32_t batch, const int32_t *prefix_slots,
                           const int64_t *prefix_off, const int32_t *new_slots, const int64_t *new_off,
                           const int32_t *new_col0, void *stream) {
    if (batch < 0 || num_rows < 0 || row_stride < 0) return SGL_ERR_INVALID;
    if (batch == 0) return SGL_OK;
    if (!r2t || !req_rows || !new_slots || !new_off) return SGL_ERR_INVALID;
    if ((prefix_slots == nullptr) != (prefix_off == nullptr)) return SGL_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    if (validate_on()) {
        std::vector<int32_t> rows, col0;
        std::vector<int64_t> poff, noff;
        if (!fetch(rows, req_rows, batch, st) || !fetch(noff, new_off, batch + 1, st)) return SGL_ERR_HIP;
        if (prefix_off && !fetch(poff, prefix_off, batch + 1, st)) return SGL_ERR_HIP;
        if (new_col0 && !fetch(col0, new_col0, batch, st)) return SGL_ERR_HIP;
        if (noff[0] != 0 || (prefix_off && poff[0] != 0)) return SGL_ERR_INVALID;
        for (int r = 0; r < batch; r++) {
            if (rows[r] < 0 || rows[r] >= num_rows) return SGL_ERR_INVALID;
            if (noff[r + 1] < noff[r]) return SGL_ERR_INVALID;
            int64_t P = 0;
            if (prefix_off) {
                if (poff[r + 1] < poff[r]) return SGL_ERR_INVALID;
                P = poff[r + 1] - poff[r];
            }
            const int64_t c0 = new_col0 ? col0[r] : P;
            if (P > row_stride || c0 < 0 || c0 + (noff[r + 1] - noff[r]) > row_stride) return SGL_ERR_INVALID;
        }
    }
    return launch_build_req_to_token(r2t, num_rows, row_stride, req_rows, batch, prefix_slots,
                                     prefix_off, new_slots, new_off, new_col0, st);
}

int sgl_count_bad_slots(const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                        const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                        uint32_t *count, void *stream) {
    if (batch < 0 || num_rows < 0 || row_stride < 0 || num_slots < 0 || max_seq_len < 0) return SGL_ERR_INVALID;
    if (batch == 0) return SGL_OK;
    if (!r2t || !req_rows || !seq_lens || !count) return SGL_ERR_INVALID;
    return launch_count_bad_slots(r2t, num_rows, row_stride, req_rows, seq_lens, batch, max_seq_len, num_slots,
                                  count, (hipStream_t)stream);
}

int sgl_store_kv(int dtype, const void *k_new, const void *v_new, int64_t n_tokens,
                 const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                 int32_t Hkv, int32_t D, void *stream) {
    if (!shape_ok(dtype, Hkv, Hkv, D)) return SGL_ERR_UNSUPPORTED;
    if (n_tokens < 0 || num_slots < 0) return SGL_ERR_INVALID;
    if (n_tokens == 0) return SGL_OK;
    if (!k_new || !v_new || !slots || !k_pool || !v_pool) return SGL_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    if (validate_on()) {
        std::vector<int32_t> s;
        if (!fetch(s, slots, (size_t)n_tokens, st)) return SGL_ERR_HIP;
        for (int32_t x : s)
            if (x < 0 || x >= num_slots) return SGL_ERR_INVALID;
    }
    return launch_store_kv(0, elt_size(dtype), k_new, v_new, n_tokens, slots, k_pool, v_pool, num_slots,
                           Hkv, D, nullptr, 0, 0, nullptr, nullptr, nullptr, 0, 0, st);
}

int sgl_store_kv_fp8(int dtype, const void *k_new, const void *v_new, int64_t n_tokens,
                     const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                     int32_t Hkv, int32_t D, const float *k_scale, const float *v_scale, void *stream) {
    if (!shape_ok(dtype, Hkv, Hkv, D)) return SGL_ERR_UNSUPPORTED;
    if (n_tokens < 0 || num_slots < 0) return SGL_ERR_INVALID;
    if (n_tokens == 0) return SGL_OK;
    if (!k_new || !v_new || !slots || !k_pool || !v_pool || !k_scale || !v_scale) return SGL_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    if (validate_on()) {
        std::vector<int32_t> s;
        if (!fetch(s, slots, (size_t)n_tokens, st)) return SGL_ERR_HIP;
        for (int32_t x : s)
            if (x < 0 || x >= num_slots) return SGL_ERR_INVALID;
    }
    return launch_store_kv_fp8(0, elt_size(dtype), k_new, v_new, n_tokens, slots, k_pool, v_pool, num_slots,
                               Hkv, D, k_scale, v_scale, nullptr, 0, 0, nullptr, nullptr, nullptr, 0, 0, st);
}

size_t sgl_extend_workspace_size(int32_t batch, int64_t n_tokens, int32_t max_extend_len, int64_t row_stride,
                                 int32_t Hq, int32_t Hkv, int32_t D) {
    if (batch <= 0 || n_tokens <= 0 || max_extend_len <= 0 || Hkv <= 0 || Hq < Hkv) return 0;
    if (small_q_extend(max_extend_len, Hq, Hkv)) return part_bytes(n_tokens, extend_splits(batch, Hkv), Hq, D);
    int32_t ksplit;
    const int32_t S = extend_key_splits(batch, max_extend_len, row_stride, Hq, Hkv, &ksplit);
    return S > 1 ? part_bytes(n_tokens, S, Hq, D) : 0;
}

int sgl_extend_attn(int dtype, const void *q, const void *k_new, const void *v_new, void *k_pool,
                    void *v_pool, int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                    int64_t row_stride, const int32_t *req_rows, const int32_t *prefix_lens,
                    const int64_t *q_off, int32_t batch, int64_t n_tokens, int32_t max_extend_len,
                    int32_t Hq, int32_t Hkv, int32_t D, float scale, void *o, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!shape_ok(dtype, Hq, Hkv, D)) return SGL_ERR_UNSUPPORTED;
    if (batch < 0 || n_tokens < 0 || max_extend_len < 0 || num_slots < 1 || num_rows < 0 || row_stride < 0)
        return SGL_ERR_INVALID;
    if (batch == 0 || n_tokens == 0) return SGL_OK;
    if (!q || !k_pool || !v_pool || !r2t || !req_rows || !prefix_lens || !q_off || !o)
        return SGL_ERR_INVALID;
    if ((k_new == nullptr) != (v_new == nullptr)) return SGL_ERR_INVALID;
    if (max_extend_len == 0) return SGL_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    if (validate_on()) {
        std::vector<int32_t> rows, plen, tab;
        std::vector<int64_t> off;
        if (!fetch(rows, req_rows, batch, st) || !fetch(plen, prefix_lens, batch, st) ||
            !fetch(off, q_off, batch + 1, st) || !fetch(tab, r2t, (size_t)(num_rows * row_stride), st))
            return SGL_ERR_HIP;
        if (off[0] != 0 || off[batch] != n_tokens) return SGL_ERR_INVALID;
        for (int r = 0; r < batch; r++) {
            const int64_t E = off[r + 1] - off[r];
            if (E < 0 || E > max_extend_len) return SGL_ERR_INVALID;
            if (rows[r] < 0 || rows[r] >= num_rows || plen[r] < 0) return SGL_ERR_INVALID;
            if (plen[r] + E > row_stride) return SGL_ERR_INVALID;
            if (!slots_ok(tab, row_stride, rows[r], 0, plen[r] + E, num_slots)) return SGL_ERR_INVALID;
        }
    }
    int rc = SGL_OK;
    if (k_new) {
        rc = launch_store_kv(1, elt_size(dtype), k_new, v_new, n_tokens, nullptr, k_pool, v_pool,
                             num_slots, Hkv, D, r2t, num_rows, row_stride, req_rows, prefix_lens,
                             q_off, batch, max_extend_len, st);
        if (rc != SGL_OK) return rc;
    }
    // The split-K path of a few new tokens per request and the key splits of
    // long prefills need workspace for their split states; with less than
    // that (or none) the call runs the prefill kernel unsplit instead: the
    // same result, only slower.  So a workspace sized for other bounds never
    // makes a call fail.
    const bool small_q_fits = workspace && workspace_bytes >= sgl_extend_workspace_size(batch, n_tokens,
                                                                                       max_extend_len, row_stride,
                                                                                       Hq, Hkv, D);
    if (dtype == SGL_BF16 && small_q_extend(max_extend_len, Hq, Hkv) && small_q_fits && n_tokens <= 0x7fffffff) {
        const int32_t n_spl = extend_splits(batch, Hkv);
        char *wp = (char *)workspace;
        SplitArgs a;
        std::memset(&a, 0, sizeof a);
        a.kind = 4; a.q = q; a.k_pool = k_pool; a.v_pool = v_pool; a.num_slots = num_slots; a.r2t = r2t;
        a.num_rows = num_rows; a.row_stride = row_stride; a.req_rows = req_rows; a.q_off = q_off;
        a.prefix_lens = prefix_lens; a.batch = batch; a.n_sets = batch; a.max_splits = n_spl; a.n_spl = n_spl;
        a.chunk = 16; a.max_members = max_extend_len; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.scale = scale;
        a.part = carve(wp, n_tokens, n_spl, Hq, D);
        if ((rc = launch_split_bf16(a, st)) != SGL_OK) return rc;
        MergeArgs m;
        std::memset(&m, 0, sizeof m);
        m.kind = 4; m.flat_or_suffix = a.part; m.batch = (int32_t)n_tokens; m.Hq = Hq; m.D = D; m.out_bf16 = 1;
        m.o = o; m.lse = lse; m.q_off = q_off; m.prefix_lens = prefix_lens; m.n_req = batch; m.n_spl = n_spl;
        return launch_merge(m, st);
    }
    if (dtype == SGL_F32)
        return launch_extend_f32((const float *)q, (const float *)k_pool, (const float *)v_pool,
                                 num_slots, r2t, num_rows, row_stride, req_rows, prefix_lens, q_off,
                                 batch, max_extend_len, Hq, Hkv, D, scale, (float *)o, lse, st);
    int32_t ksplit;
    int32_t n_split = extend_key_splits(batch, max_extend_len, row_stride, Hq, Hkv, &ksplit);
    if (n_split > 1 && (!workspace || workspace_bytes < part_bytes(n_tokens, n_split, Hq, D) || n_tokens > 0x7fffffff))
        n_split = 1;
    if (n_split <= 1) {
        PartialBuf none;
        std::memset(&none, 0, sizeof none);
        return launch_extend_bf16((const __bf16 *)q, (const __bf16 *)k_pool, (const __bf16 *)v_pool, num_slots, r2t,
                                  num_rows, row_stride, req_rows, prefix_lens, q_off, batch, max_extend_len, Hq, Hkv,
                                  D, scale, (__bf16 *)o, lse, 1, 0, none, st);
    }
    char *wp = (char *)workspace;
    const PartialBuf part = carve(wp, n_tokens, n_split, Hq, D);
    if ((rc = launch_extend_bf16((const __bf16 *)q, (const __bf16 *)k_pool, (const __bf16 *)v_pool, num_slots, r2t,
                                 num_rows, row_stride, req_rows, prefix_lens, q_off, batch, max_extend_len, Hq, Hkv, D,
                                 scale, nullptr, nullptr, n_split, ksplit, part, st)) != SGL_OK)
        return rc;
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    m.kind = 5; m.flat_or_suffix = part; m.batch = (int32_t)n_tokens; m.Hq = Hq; m.Hkv = Hkv; m.D = D;
    m.out_bf16 = 1; m.o = o; m.lse = lse; m.q_off = q_off; m.prefix_lens = prefix_lens; m.n_req = batch;
    m.chunk_flat = ksplit; m.row_stride = row_stride;
    return launch_merge(m, st);
}

// Splits of the flat call and the cascade suffix are sized for the smaller
// split of the two kernels that may run them.
size_t sgl_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t Hq, int32_t Hkv, int32_t D) {
    (void)Hkv;
    if (batch <= 0 || max_seq_len <= 0) return 0;
    const int64_t S = ceil_div64(max_seq_len, kRowsChunk);
    return part_bytes(batch, S, Hq, D);
}

namespace {

int decode_common(bool cascade, bool fp8, int dtype, const void *q, const void *k_new, const void *v_new,
                  void *k_pool, void *v_pool, const float *k_scale, const float *v_scale, int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                  int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                  const int32_t *group_ptr, const int32_t *group_prefix_len, int32_t batch, int32_t G,
                  int32_t max_seq_len, int32_t max_group_size, int32_t max_prefix_len, int32_t Hq,
                  int32_t Hkv, int32_t D, float scale, void *o, float *lse, void *workspace,
                  size_t workspace_bytes, void *stream) {
    if (!shape_ok(dtype, Hq, Hkv, D)) return SGL_ERR_UNSUPPORTED;
    if (fp8 && dtype != SGL_BF16) return SGL_ERR_UNSUPPORTED;   // FP8 KV: bf16 queries only
    if (batch < 0 || max_seq_len < 0 || num_slots < 1 || num_rows < 0 || row_stride < 0)
        return SGL_ERR_INVALID;
    if (batch == 0) return SGL_OK;
    if (!q || !k_pool || !v_pool || !r2t || !req_rows || !seq_lens || !o) return SGL_ERR_INVALID;
    if (fp8 && (!k_scale || !v_scale)) return SGL_ERR_INVALID;
    if ((k_new == nullptr) != (v_new == nullptr)) return SGL_ERR_INVALID;
    if (max_seq_len < 1) return SGL_ERR_INVALID;
    const int g = Hq / Hkv;
    if (cascade) {
        if (G < 1 || G > batch || !group_ptr || !group_prefix_len) return SGL_ERR_INVALID;
        if (max_group_size < 1 || max_prefix_len < 0 || max_prefix_len > max_seq_len) return SGL_ERR_INVALID;
        if ((int64_t)max_group_size * g > 4096) return SGL_ERR_UNSUPPORTED;
    }
    // Kernel choice (measured on the 256-request decode workload):
    //  - cascade suffix: whole-row loads, work dealt to the XCDs set by set
    //    (the suffixes share nothing, so balance matters most);
    //  - flat fp8: whole-row loads with blocks of kFlatXcdBlock consecutive
    //    requests per XCD, so siblings share prefix rows through one L2;
    //  - flat bf16: the per-head kernel, whose head-per-XCD order already gets
    //    that reuse with every XCD holding an equal share of each request (the
    //    whole-row kernel here measured mixed: faster on the fork, 241 -> 214
    //    us, and on chunked-prefill decode with 16-token pages, 7.61 -> 7.52 ms
    //    per run, slower on 256 requests with no shared prefix, 1,028 -> 1,061
    //    us, and within noise on the decode workload);
    //  - other shapes, and the cascade prefix stage: the per-head kernels.
    const bool rows_ok = dtype != SGL_F32 && (Hkv == 2 || Hkv == 4 || Hkv == 8 || Hkv == 16) && g <= 16;
    const bool rows_flat = rows_ok && fp8;
    const bool rows_suffix = rows_ok;
    // Cascade suffix stage in equal runs of the concatenated suffixes, the
    // prefix items behind them in the same grid (launch_cascade_balanced),
    // for D 128 with KV heads in groups of 4 and suffixes of about a suffix
    // split or more.  On the 256-request decode workload the call takes
    // 576-580 us this way against 618-625 us with the one grid of split items
    // (FP8 cache: 336-337 against 343-345 us), and 586 us with the prefix
    // stage in a launch of its own before the runs (600 us with the prefix
    // items first in the grid).  Shorter suffixes would cut a run into many
    // one-request pieces, each paying its own start (the 8-branch fork: 122
    // against 75 us at one key), so those keep the split items.
    const bool balanced = cascade && rows_suffix && D == 128 && Hkv % 4 == 0 && max_prefix_len > 0 &&
                          (int64_t)max_seq_len - max_prefix_len >= kSuffixChunk;
    const int32_t sk_wgs = (int32_t)balanced_wgs(Hkv);
    // Split sizes.  The cascade's preferred prefix and suffix splits depend on
    // the call's bounds (smaller bounds can prefer smaller splits, hence more
    // split states), so they are doubled, up to kPrefixChunkMax and
    // kSuffixChunk keys, while their states would not fit the caller's
    // workspace: a workspace sized by sgl_cascade_workspace_size for larger
    // bounds always holds splits of those sizes.
    int pchunk = kPrefixChunkMax, fchunk = rows_flat ? kRowsChunk : kDecodeChunk;
    size_t need;
    if (cascade) {
        pchunk = prefix_chunk(G, max_group_size, max_prefix_len, Hq, Hkv, D);
        fchunk = rows_suffix ? suffix_chunk(batch, max_seq_len, max_prefix_len, Hkv) : kDecodeChunk;
        auto need_for = [&](int pc, int fc) {
            const int64_t Sp = max_prefix_len > 0 ? ceil_div64(max_prefix_len, pc) : 1;
            return part_bytes(batch, Sp, Hq, D) + suffix_part_bytes(batch, ceil_div64(max_seq_len, fc), Hq, Hkv, D) +
                   align_up((size_t)batch * sizeof(int32_t)) + align_up((size_t)(batch + 2) * sizeof(int64_t));
        };
        while (need_for(pchunk, fchunk) > workspace_bytes) {
            if (fchunk < kSuffixChunk && (fchunk <= pchunk || pchunk >= kPrefixChunkMax)) fchunk *= 2;
            else if (pchunk < kPrefixChunkMax) pchunk *= 2;
            else break;
        }
        need = need_for(pchunk, fchunk);
    } else {
        need = sgl_decode_workspace_size(batch, max_seq_len, Hq, Hkv, D);
    }
    if (workspace_bytes < need || (need > 0 && !workspace)) return SGL_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;

    if (validate_on()) {
        std::vector<int32_t> rows, lens, tab, gptr, gpl;
        if (!fetch(rows, req_rows, batch, st) || !fetch(lens, seq_lens, batch, st) ||
            !fetch(tab, r2t, (size_t)(num_rows * row_stride), st))
            return SGL_ERR_HIP;
        for (int r = 0; r < batch; r++) {
            if (rows[r] < 0 || rows[r] >= num_rows) return SGL_ERR_INVALID;
            if (lens[r] < 1 || lens[r] > max_seq_len || lens[r] > row_stride) return SGL_ERR_INVALID;
            if (!slots_ok(tab, row_stride, rows[r], 0, lens[r], num_slots)) return SGL_ERR_INVALID;
        }
        if (cascade) {
            if (!fetch(gptr, group_ptr, G + 1, st) || !fetch(gpl, group_prefix_len, G, st)) return SGL_ERR_HIP;
            if (gptr[0] != 0 || gptr[G] != batch) return SGL_ERR_INVALID;
            for (int gg = 0; gg < G; gg++) {
                const int a = gptr[gg], b = gptr[gg + 1];
                if (b <= a || b - a > max_group_size) return SGL_ERR_INVALID;
                if (gpl[gg] < 0 || gpl[gg] > max_prefix_len) return SGL_ERR_INVALID;
                for (int r = a; r < b; r++) {
                    if (gpl[gg] > lens[r] || (k_new && gpl[gg] >= lens[r])) return SGL_ERR_INVALID;
                    if (std::memcmp(&tab[(size_t)rows[r] * row_stride], &tab[(size_t)rows[a] * row_stride],
                                    sizeof(int32_t) * (size_t)gpl[gg]) != 0)
                        return SGL_ERR_INVALID;
                }
                if (k_new && gpl[gg] > 0) {   // the stored tokens' slots lie outside the prefix
                    const int32_t *pre = &tab[(size_t)rows[a] * row_stride];
                    std::vector<int32_t> sorted(pre, pre + gpl[gg]);
                    std::sort(sorted.begin(), sorted.end());
                    for (int r = a; r < b; r++)
                        if (std::binary_search(sorted.begin(), sorted.end(),
                                               tab[(size_t)rows[r] * row_stride + lens[r] - 1]))
                            return SGL_ERR_INVALID;
                }
            }
        }
    }

    // Workspace: [flat splits] or [prefix splits][suffix splits][suffix starts]
    char *wp = (char *)workspace;
    const int64_t Sp = max_prefix_len > 0 ? ceil_div64(max_prefix_len, pchunk) : 1;
    const int64_t Ss = ceil_div64(max_seq_len, fchunk);
    PartialBuf flat_part{}, pre_part{}, suf_part{};
    int32_t *suffix_lo = nullptr;
    int64_t *sk_plan = nullptr;
    if (!cascade) {
        flat_part = carve(wp, batch, ceil_div64(max_seq_len, fchunk), Hq, D);
    } else {
        pre_part = carve(wp, batch, Sp, Hq, D);
        char *suf_base = wp;
        suf_part = carve(wp, batch, Ss, Hq, D);
        wp = suf_base + suffix_part_bytes(batch, Ss, Hq, Hkv, D);
        suffix_lo = (int32_t *)wp;
        wp += align_up((size_t)batch * sizeof(int32_t));
        sk_plan = (int64_t *)wp;
        if (balanced) {   // the same bytes as batch + sk_wgs state rows of one split each
            char *b = suf_base;
            suf_part = carve(b, sk_state_rows(batch, sk_wgs), 1, Hq, D);
        }
    }
    // Both cascade stages in one grid when the shape allows it (D 128, KV
    // heads in groups of 4) and the suffix items are the longer ones: a
    // suffix item walks fchunk / 16 tiles one at a time, a prefix item
    // pchunk / 16 tiles with three in flight, so that is 3 fchunk > pchunk.
    // The suffix rounds that suffixes of about max_seq_len - max_prefix_len
    // keys need (twice that, for groups with shorter prefixes) go first, the
    // prefix items fill the compute units as they run out, and the rest of
    // the Ss rounds (mostly empty) go last.  Measured: the 256-request decode
    // workload takes 651 us this way against 666 us in two launches; on the
    // 8-branch fork (prefix items longer) one grid with the prefix items
    // first loses to two launches as the suffixes grow (139 against 129 us at
    // 512 keys), so such calls keep one launch per stage.
    const bool one_grid = !balanced && cascade && max_prefix_len > 0 && rows_suffix && D == 128 && Hkv % 4 == 0 &&
                          3 * fchunk > pchunk;
    // The current token's K/V, and (cascade) each request's suffix start,
    // found once for every suffix item and the merge.  A bf16-query cascade
    // call in two launches hands both to the leading workgroups of its
    // prefix-stage launch (the prefix items never read a current token:
    // every group prefix ends before its requests' current positions);
    // otherwise they take a kernel of their own before the attention.
    SuffixStartArgs ss;
    std::memset(&ss, 0, sizeof ss);
    ss.group_ptr = group_ptr; ss.group_prefix_len = group_prefix_len; ss.seq_lens = seq_lens;
    ss.G = G; ss.batch = batch; ss.lo = suffix_lo;
    if (balanced) {   // and the balanced stage's plan, by one more workgroup of the same launch
        ss.plan = sk_plan; ss.plan_wgs = sk_wgs; ss.req_rows = req_rows; ss.num_rows = num_rows;
        ss.row_stride = row_stride;
    }
    const bool carry_store = cascade && max_prefix_len > 0 && !one_grid && !balanced && dtype == SGL_BF16;
    int rc = SGL_OK;
    if (carry_store) {
        // launched with the prefix stage below
    } else if (k_new) {
        const SuffixStartArgs *ssp = cascade ? &ss : nullptr;
        rc = fp8 ? launch_store_kv_fp8(2, elt_size(dtype), k_new, v_new, batch, nullptr, k_pool, v_pool,
                                       num_slots, Hkv, D, k_scale, v_scale, r2t, num_rows, row_stride,
                                       req_rows, seq_lens, nullptr, batch, 0, st, ssp)
                 : launch_store_kv(2, elt_size(dtype), k_new, v_new, batch, nullptr, k_pool, v_pool, num_slots,
                                   Hkv, D, r2t, num_rows, row_stride, req_rows, seq_lens, nullptr, batch, 0, st,
                                   ssp);
    } else if (cascade) {
        rc = launch_suffix_start(ss, st);
    }
    if (rc != SGL_OK) return rc;

    SplitArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k_pool = k_pool; a.v_pool = v_pool; a.num_slots = num_slots; a.r2t = r2t;
    a.num_rows = num_rows; a.row_stride = row_stride; a.req_rows = req_rows; a.seq_lens = seq_lens;
    a.group_ptr = group_ptr; a.group_prefix_len = group_prefix_len; a.batch = batch; a.G = G;
    a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.scale = scale; a.k_scale = k_scale; a.v_scale = v_scale;
    auto run_split = [&](const SplitArgs &x, bool rows) {
        if (dtype == SGL_F32) return launch_split_f32(x, st);
        if (rows) {
            SplitArgs y = x;
            y.xcd_block = x.kind == 2 ? 1 : kFlatXcdBlock;
            return launch_split_rows(y, fp8, st);
        }
        return fp8 ? launch_split_fp8(x, st) : launch_split_bf16(x, st);
    };

    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    m.seq_lens = seq_lens; m.group_ptr = group_ptr; m.group_prefix_len = group_prefix_len;
    m.batch = batch; m.G = G; m.Hq = Hq; m.D = D; m.out_bf16 = dtype == SGL_BF16; m.o = o; m.lse = lse;
    m.chunk_flat = fchunk; m.chunk_prefix = pchunk;

    if (!cascade) {
        a.kind = 0; a.n_sets = batch; a.max_splits = (int32_t)flat_part.S; a.chunk = fchunk;
        a.part = flat_part;
        if ((rc = run_split(a, rows_flat)) != SGL_OK) return rc;
        m.kind = 0; m.flat_or_suffix = a.part;
        return launch_merge(m, st);
    }
    SplitArgs pa = a;
    pa.kind = 1; pa.chunk = pchunk; pa.max_splits = (int32_t)Sp; pa.max_members = max_group_size;
    pa.part = pre_part;
    // the f32 path walks (request, head, split) for every kind; the bf16 path one wave per group
    pa.n_sets = dtype == SGL_F32 ? batch : G;
    SplitArgs sa = a;
    sa.kind = 2; sa.chunk = fchunk; sa.max_splits = (int32_t)Ss; sa.n_sets = batch;
    sa.part = suf_part;
    sa.suffix_lo = suffix_lo;
    m.suffix_lo = suffix_lo;

    if (carry_store)
        pa.store = decode_store_args(elt_size(dtype), fp8, k_new, v_new, batch, k_pool, v_pool, num_slots, Hkv, D,
                                     k_scale, v_scale, r2t, num_rows, row_stride, req_rows, seq_lens, &ss);
    // Suffix split rounds for suffixes of about max_seq_len - max_prefix_len
    // keys, twice that for groups with shorter prefixes: the rest of the Ss
    // rounds, mostly empty, go after the prefix items in one grid; in two
    // launches (whole-row suffix kernel) the grid holds only these rounds
    // and its workgroups take the later rounds' items that have keys (on the
    // fork, 65 rounds of 64-key splits for suffixes of one key otherwise
    // dispatch some 16,000 empty workgroups).
    const int64_t est = std::max<int64_t>(1, (int64_t)max_seq_len - max_prefix_len);
    const int32_t head = (int32_t)std::min<int64_t>(Ss, 2 * ceil_div64(est, fchunk));
    if (balanced) {
        SplitArgs sx = sa;
        sx.sk_wgs = sk_wgs;
        sx.chunk = kSuffixChunk;
        sx.sk_plan = sk_plan;
        if ((rc = launch_cascade_balanced(pa, sx, fp8, st)) != SGL_OK) return rc;
        m.sk_plan = sk_plan;
    } else if (one_grid) {
        SplitArgs sx = sa;
        sx.xcd_block = 1;
        if ((rc = launch_cascade_split(pa, sx, head, fp8, st)) != SGL_OK) return rc;
    } else {
        if (max_prefix_len > 0 && (rc = run_split(pa, false)) != SGL_OK) return rc;
        SplitArgs sx = sa;
        if (rows_suffix && dtype != SGL_F32) sx.rounds = head;
        if ((rc = run_split(sx, rows_suffix)) != SGL_OK) return rc;
    }
    m.kind = 3; m.prefix = pa.part; m.flat_or_suffix = sa.part;
    if (max_prefix_len == 0) m.kind = 0, m.flat_or_suffix = sa.part;
    return launch_merge(m, st);
}

}  // namespace

int sgl_decode_attn(int dtype, const void *q, const void *k_new, const void *v_new, void *k_pool,
                    void *v_pool, int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                    int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens, int32_t batch,
                    int32_t max_seq_len, int32_t Hq, int32_t Hkv, int32_t D, float scale, void *o,
                    float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(false, false, dtype, q, k_new, v_new, k_pool, v_pool, nullptr, nullptr, num_slots,
                         r2t, num_rows, row_stride, req_rows, seq_lens, nullptr, nullptr, batch, 0,
                         max_seq_len, 0, 0, Hq, Hkv, D, scale, o, lse, workspace, workspace_bytes, stream);
}

int sgl_decode_attn_fp8kv(int dtype, const void *q, const void *k_new, const void *v_new, void *k_pool,
                          void *v_pool, const float *k_scale, const float *v_scale, int64_t num_slots,
                          const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                          const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int32_t Hq,
                          int32_t Hkv, int32_t D, float scale, void *o, float *lse, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return decode_common(false, true, dtype, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, num_slots,
                         r2t, num_rows, row_stride, req_rows, seq_lens, nullptr, nullptr, batch, 0,
                         max_seq_len, 0, 0, Hq, Hkv, D, scale, o, lse, workspace, workspace_bytes, stream);
}

size_t sgl_cascade_workspace_size(int32_t batch, int32_t G, int32_t max_seq_len, int32_t max_group_size,
                                  int32_t max_prefix_len, int32_t Hq, int32_t Hkv, int32_t D) {
    if (batch <= 0 || max_seq_len <= 0) return 0;
    if (G < 1 || Hkv < 1 || Hq < Hkv || max_group_size < 1) return 0;
    const int64_t Sp = max_prefix_len > 0
                           ? ceil_div64(max_prefix_len, prefix_chunk(G, max_group_size, max_prefix_len, Hq, Hkv, D))
                           : 1;
    const int64_t Ss = ceil_div64(max_seq_len, suffix_chunk(batch, max_seq_len, max_prefix_len, Hkv));
    // split states of both stages, each request's suffix start, the balanced suffix stage's plan
    return part_bytes(batch, Sp, Hq, D) + suffix_part_bytes(batch, Ss, Hq, Hkv, D) +
           align_up((size_t)batch * sizeof(int32_t)) + align_up((size_t)(batch + 2) * sizeof(int64_t));
}

int sgl_cascade_decode_attn(int dtype, const void *q, const void *k_new, const void *v_new, void *k_pool,
                            void *v_pool, int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                            int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                            const int32_t *group_ptr, const int32_t *group_prefix_len, int32_t batch,
                            int32_t G, int32_t max_seq_len, int32_t max_group_size,
                            int32_t max_prefix_len, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                            void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(true, false, dtype, q, k_new, v_new, k_pool, v_pool, nullptr, nullptr, num_slots,
                         r2t, num_rows, row_stride, req_rows, seq_lens, group_ptr, group_prefix_len, batch,
                         G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D, scale, o, lse,
                         workspace, workspace_bytes, stream);
}

// ---- allocation-free cascade decode ---------------------------------------------
// The split states of sgl_cascade_decode_attn_static live in a fixed device
// array that each GPU the library runs on holds until the process ends.  In
// host code the array's name is a host-side stand-in, not a device address:
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address reaches the kernels.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch_addr[kMaxDevices];

// The current device's address of `scratch` (looked up on its first use).
static int static_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SGL_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SGL_ERR_UNSUPPORTED;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return SGL_ERR_HIP;
        }
        g_scratch_addr[dev].store(p, std::memory_order_release);   // racing threads store the same address
    }
    *out = p;
    return SGL_OK;
}

size_t sgl_static_scratch_bytes(void) { return kStaticScratchBytes; }

int sgl_cascade_decode_attn_static(int dtype, const void *q, const void *k_new, const void *v_new, void *k_pool,
                                   void *v_pool, int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                                   int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                                   const int32_t *group_ptr, const int32_t *group_prefix_len, int32_t batch,
                                   int32_t G, int32_t max_seq_len, int32_t max_group_size,
                                   int32_t max_prefix_len, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                   void *o, float *lse, void *stream) {
    void *ws = nullptr;
    const int rc = static_scratch(&ws);
    if (rc != SGL_OK) return rc;
    return decode_common(true, false, dtype, q, k_new, v_new, k_pool, v_pool, nullptr, nullptr, num_slots,
                         r2t, num_rows, row_stride, req_rows, seq_lens, group_ptr, group_prefix_len, batch,
                         G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D, scale, o, lse,
                         ws, kStaticScratchBytes, stream);
}

int sgl_cascade_decode_attn_fp8kv(int dtype, const void *q, const void *k_new, const void *v_new,
                                  void *k_pool, void *v_pool, const float *k_scale, const float *v_scale,
                                  int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                                  int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                                  const int32_t *group_ptr, const int32_t *group_prefix_len, int32_t batch,
                                  int32_t G, int32_t max_seq_len, int32_t max_group_size,
                                  int32_t max_prefix_len, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                  void *o, float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    return decode_common(true, true, dtype, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, num_slots,
                         r2t, num_rows, row_stride, req_rows, seq_lens, group_ptr, group_prefix_len, batch,
                         G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D, scale, o, lse,
                         workspace, workspace_bytes, stream);
}

// ---- MLA latent decode ---------------------------------------------------------
size_t sgl_mla_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t Hq, int32_t Dv) {
    if (batch <= 0 || max_seq_len <= 0 || Hq <= 0 || Dv <= 0) return 0;
    return part_bytes(batch, ceil_div64(max_seq_len, mla_chunk(Hq)), Hq, Dv);
}

size_t sgl_mla_cascade_workspace_size(int32_t batch, int32_t G, int32_t max_seq_len, int32_t max_group_size,
                                      int32_t max_prefix_len, int32_t Hq, int32_t Dv) {
    if (batch <= 0 || max_seq_len <= 0 || G < 1 || max_group_size < 1 || Hq <= 0 || Dv <= 0) return 0;
    const int64_t Sp = max_prefix_len > 0
                           ? ceil_div64(max_prefix_len, mla_prefix_chunk(G, max_group_size, max_prefix_len, Hq))
                           : 1;
    return part_bytes(batch, Sp, Hq, Dv) + part_bytes(batch, ceil_div64(max_seq_len, mla_chunk(Hq)), Hq, Dv);
}

namespace {

int mla_common(bool cascade, const void *q, const void *kv_new, void *kv_pool, int64_t num_slots,
               const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
               const int32_t *seq_lens, const int32_t *group_ptr, const int32_t *group_prefix_len, int32_t batch,
               int32_t G, int32_t max_seq_len, int32_t max_group_size, int32_t max_prefix_len, int32_t Hq,
               int32_t Dqk, int32_t Dv, float scale, void *o, float *lse, void *workspace, size_t workspace_bytes,
               void *stream) {
    if (Dqk != kMlaDqk || Dv != kMlaDv || Hq < 16 || Hq % 16 != 0 || Hq > 128) return SGL_ERR_UNSUPPORTED;
    if (batch < 0 || max_seq_len < 0 || num_slots < 1 || num_rows < 0 || row_stride < 0) return SGL_ERR_INVALID;
    if (batch == 0) return SGL_OK;
    if (!q || !kv_pool || !r2t || !req_rows || !seq_lens || !o || max_seq_len < 1) return SGL_ERR_INVALID;
    if (cascade) {
        if (G < 1 || G > batch || !group_ptr || !group_prefix_len) return SGL_ERR_INVALID;
        if (max_group_size < 1 || max_prefix_len < 0 || max_prefix_len > max_seq_len) return SGL_ERR_INVALID;
        if ((int64_t)max_group_size * Hq > 4096) return SGL_ERR_UNSUPPORTED;
    }
    // A prefix-stage workgroup holds at most 64 query rows and reads the shared
    // prefix once for them; a group with more rows would read it once per 64
    // rows from workgroups of 16 waves, which measured slower than reading it
    // once per request (128 requests in groups of 8 over 2-8k keys: 16 heads
    // 253 vs 208 us, 128 heads 885 vs 805 us), and so did a prefix item per
    // group whose 64-row workgroups share each tile through one XCD's L2
    // (16 heads 196-214 vs 188 us, 128 heads 479-507 vs 405-413 us: the
    // per-request prefix states and the merge cost more than the re-reads).
    // Such groups run the flat splits (same result) and need only the flat
    // call's workspace.
    const bool flat_path = !cascade || (int64_t)max_group_size * Hq > 64;
    const int chunk = mla_chunk(Hq);
    const int64_t Ss = ceil_div64(max_seq_len, chunk);
    // The preferred prefix split depends on the call's bounds (a shorter
    // prefix can prefer a smaller split, hence more split states), so it is
    // doubled, up to 512 keys, while the states would not fit the caller's
    // workspace: a workspace sized by sgl_mla_cascade_workspace_size for
    // larger bounds always holds 512-key splits.
    int pchunk = kPrefixChunkMax;
    size_t need;
    if (flat_path) {
        need = sgl_mla_decode_workspace_size(batch, max_seq_len, Hq, Dv);
    } else {
        pchunk = mla_prefix_chunk(G, max_group_size, max_prefix_len, Hq);
        auto need_for = [&](int pc) {
            const int64_t Sp = max_prefix_len > 0 ? ceil_div64(max_prefix_len, pc) : 1;
            return part_bytes(batch, Sp, Hq, Dv) + part_bytes(batch, Ss, Hq, Dv);
        };
        while (need_for(pchunk) > workspace_bytes && pchunk < kPrefixChunkMax) pchunk *= 2;
        need = need_for(pchunk);
    }
    if (workspace_bytes < need || (need > 0 && !workspace)) return SGL_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (validate_on()) {
        std::vector<int32_t> rows, lens, tab, gptr, gpl;
        if (!fetch(rows, req_rows, batch, st) || !fetch(lens, seq_lens, batch, st) ||
            !fetch(tab, r2t, (size_t)(num_rows * row_stride), st))
            return SGL_ERR_HIP;
        for (int r = 0; r < batch; r++) {
            if (rows[r] < 0 || rows[r] >= num_rows) return SGL_ERR_INVALID;
            if (lens[r] < 1 || lens[r] > max_seq_len || lens[r] > row_stride) return SGL_ERR_INVALID;
            if (!slots_ok(tab, row_stride, rows[r], 0, lens[r], num_slots)) return SGL_ERR_INVALID;
        }
        if (cascade) {
            if (!fetch(gptr, group_ptr, G + 1, st) || !fetch(gpl, group_prefix_len, G, st)) return SGL_ERR_HIP;
            if (gptr[0] != 0 || gptr[G] != batch) return SGL_ERR_INVALID;
            for (int gg = 0; gg < G; gg++) {
                const int a = gptr[gg], b = gptr[gg + 1];
                if (b <= a || b - a > max_group_size || gpl[gg] < 0 || gpl[gg] > max_prefix_len) return SGL_ERR_INVALID;
                for (int r = a; r < b; r++) {
                    if (gpl[gg] > lens[r]) return SGL_ERR_INVALID;
                    if (std::memcmp(&tab[(size_t)rows[r] * row_stride], &tab[(size_t)rows[a] * row_stride],
                                    sizeof(int32_t) * (size_t)gpl[gg]) != 0)
                        return SGL_ERR_INVALID;
                }
            }
        }
    }
    int rc = SGL_OK;
    if (kv_new) {   // one latent pool: the same rows serve as K and V
        rc = launch_store_kv(2, 2, kv_new, kv_new, batch, nullptr, kv_pool, kv_pool, num_slots, 1, Dqk, r2t,
                             num_rows, row_stride, req_rows, seq_lens, nullptr, batch, 0, st);
        if (rc != SGL_OK) return rc;
    }
    char *wp = (char *)workspace;
    SplitArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k_pool = kv_pool; a.v_pool = kv_pool; a.num_slots = num_slots; a.r2t = r2t;
    a.num_rows = num_rows; a.row_stride = row_stride; a.req_rows = req_rows; a.seq_lens = seq_lens;
    a.group_ptr = group_ptr; a.group_prefix_len = group_prefix_len; a.batch = batch; a.G = G;
    a.Hq = Hq; a.Hkv = 1; a.D = Dqk; a.scale = scale;
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    m.seq_lens = seq_lens; m.group_ptr = group_ptr; m.group_prefix_len = group_prefix_len;
    m.batch = batch; m.G = G; m.Hq = Hq; m.D = Dv; m.out_bf16 = 1; m.o = o; m.lse = lse;
    m.chunk_flat = chunk;
    if (flat_path) {
        a.kind = 0; a.n_sets = batch; a.max_splits = (int32_t)Ss; a.chunk = chunk;
        a.part = carve(wp, batch, Ss, Hq, Dv);
        if ((rc = launch_split_mla(a, st)) != SGL_OK) return rc;
        m.kind = 0; m.flat_or_suffix = a.part;
        return launch_merge(m, st);
    }
    const int64_t Sp = max_prefix_len > 0 ? ceil_div64(max_prefix_len, pchunk) : 1;
    SplitArgs pa = a;
    pa.kind = 1; pa.chunk = pchunk; pa.max_splits = (int32_t)Sp; pa.max_members = max_group_size; pa.n_sets = G;
    pa.part = carve(wp, batch, Sp, Hq, Dv);
    SplitArgs sa = a;
    sa.kind = 2; sa.chunk = chunk; sa.max_splits = (int32_t)Ss; sa.n_sets = batch;
    sa.part = carve(wp, batch, Ss, Hq, Dv);
    if (max_prefix_len > 0 && (rc = launch_split_mla(pa, st)) != SGL_OK) return rc;
    if ((rc = launch_split_mla(sa, st)) != SGL_OK) return rc;
    m.chunk_prefix = pchunk;
    m.kind = max_prefix_len > 0 ? 3 : 0; m.prefix = pa.part; m.flat_or_suffix = sa.part;
    return launch_merge(m, st);
}

}  // namespace

int sgl_mla_decode_attn(const void *q, const void *kv_new, void *kv_pool, int64_t num_slots, const int32_t *r2t,
                        int64_t num_rows, int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                        int32_t batch, int32_t max_seq_len, int32_t Hq, int32_t Dqk, int32_t Dv, float scale,
                        void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    return mla_common(false, q, kv_new, kv_pool, num_slots, r2t, num_rows, row_stride, req_rows, seq_lens, nullptr,
                      nullptr, batch, 0, max_seq_len, 0, 0, Hq, Dqk, Dv, scale, o, lse, workspace, workspace_bytes,
                      stream);
}

int sgl_mla_cascade_decode_attn(const void *q, const void *kv_new, void *kv_pool, int64_t num_slots,
                                const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                                const int32_t *seq_lens, const int32_t *group_ptr, const int32_t *group_prefix_len,
                                int32_t batch, int32_t G, int32_t max_seq_len, int32_t max_group_size,
                                int32_t max_prefix_len, int32_t Hq, int32_t Dqk, int32_t Dv, float scale, void *o,
                                float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    return mla_common(true, q, kv_new, kv_pool, num_slots, r2t, num_rows, row_stride, req_rows, seq_lens, group_ptr,
                      group_prefix_len, batch, G, max_seq_len, max_group_size, max_prefix_len, Hq, Dqk, Dv, scale,
                      o, lse, workspace, workspace_bytes, stream);
}

namespace {

// The device-visible address of a caller's host-tier buffer, after checking
// that every one of its `bytes` bytes is page-locked host memory mapped for
// the device (a kernel touching pageable memory would fault).
int host_tier_addr(const void *p, size_t bytes, char **dev) {
    hipPointerAttribute_t a, b;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return SGL_ERR_INVALID;
    }
    if (a.type != hipMemoryTypeHost || a.devicePointer == nullptr) return SGL_ERR_INVALID;
    if (hipPointerGetAttributes(&b, (const char *)p + (bytes - 1)) != hipSuccess) {
        (void)hipGetLastError();
        return SGL_ERR_INVALID;
    }
    if (b.type != hipMemoryTypeHost || (char *)b.devicePointer != (char *)a.devicePointer + (bytes - 1))
        return SGL_ERR_INVALID;
    *dev = (char *)a.devicePointer;
    return SGL_OK;
}

// dir 0: host rows -> pool slots; dir 1: pool slots -> host rows.
int hicache_move(int dir, const void *host_k, const void *host_v, int64_t n_host_rows, const int64_t *host_rows,
                 const int32_t *slots, int64_t n, const void *k_pool, const void *v_pool, int64_t num_slots,
                 int64_t row_bytes, hipStream_t st) {
    if (n < 0 || n_host_rows < 0 || num_slots < 0 || row_bytes <= 0 || row_bytes % 16 != 0) return SGL_ERR_INVALID;
    if (n == 0) return SGL_OK;
    if (!host_k || !k_pool || !host_rows || !slots || n_host_rows == 0 || num_slots == 0) return SGL_ERR_INVALID;
    if ((host_v == nullptr) != (v_pool == nullptr)) return SGL_ERR_INVALID;
    if (((uintptr_t)host_k | (uintptr_t)host_v | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15) return SGL_ERR_INVALID;
    if (n_host_rows > INT64_MAX / row_bytes || num_slots > INT64_MAX / row_bytes) return SGL_ERR_INVALID;
    const size_t bytes = (size_t)(n_host_rows * row_bytes);
    char *hk = nullptr, *hv = nullptr;
    int rc;
    if ((rc = host_tier_addr(host_k, bytes, &hk)) != SGL_OK) return rc;
    if (host_v && (rc = host_tier_addr(host_v, bytes, &hv)) != SGL_OK) return rc;
    if (validate_on()) {
        std::vector<int64_t> h;
        std::vector<int32_t> s;
        if (!fetch(h, host_rows, (size_t)n, st) || !fetch(s, slots, (size_t)n, st)) return SGL_ERR_HIP;
        std::vector<int64_t> dst(n);
        for (int64_t i = 0; i < n; ++i) {
            if (h[i] < 0 || h[i] >= n_host_rows || s[i] < 0 || s[i] >= num_slots) return SGL_ERR_INVALID;
            dst[i] = dir == 0 ? s[i] : h[i];
        }
        std::sort(dst.begin(), dst.end());
        if (std::adjacent_find(dst.begin(), dst.end()) != dst.end()) return SGL_ERR_INVALID;
    }
    MoveArgs a;
    const char *pk = (const char *)k_pool, *pv = (const char *)v_pool;
    a.src[0] = dir == 0 ? hk : pk;
    a.src[1] = dir == 0 ? hv : pv;
    a.dst[0] = dir == 0 ? (char *)pk : hk;
    a.dst[1] = dir == 0 ? (char *)pv : hv;
    a.host_rows = host_rows;
    a.slots = slots;
    a.n = n;
    a.n_host_rows = n_host_rows;
    a.num_slots = num_slots;
    a.row_bytes = row_bytes;
    a.cpr = row_bytes / 16;
    a.n_t = host_v ? 2 : 1;
    return launch_move_rows(dir, a, st);
}

}  // namespace

int sgl_hicache_prefetch(const void *host_k, const void *host_v, int64_t n_host_rows, const int64_t *host_rows,
                         const int32_t *slots, int64_t n, void *k_pool, void *v_pool, int64_t num_slots,
                         int64_t row_bytes, void *stream) {
    return hicache_move(0, host_k, host_v, n_host_rows, host_rows, slots, n, k_pool, v_pool, num_slots, row_bytes,
                        (hipStream_t)stream);
}

int sgl_hicache_write_back(const void *k_pool, const void *v_pool, int64_t num_slots, const int32_t *slots,
                           const int64_t *host_rows, int64_t n, void *host_k, void *host_v, int64_t n_host_rows,
                           int64_t row_bytes, void *stream) {
    return hicache_move(1, host_k, host_v, n_host_rows, host_rows, slots, n, k_pool, v_pool, num_slots, row_bytes,
                        (hipStream_t)stream);
}

}  // extern "C"
