// common.h -- internal helpers shared by the HIP sources of libsgl_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgl_attn.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define SGL_LDS __attribute__((address_space(3)))

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Split key-index range helpers --------------------------------------------
__host__ __device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A slot read from req_to_token is used only if it lies in the pool.
__device__ __forceinline__ int32_t safe_slot(int32_t s, int64_t num_slots) {
    return (s >= 0 && (int64_t)s < num_slots) ? s : 0;
}

// Prefix group of request r: the last g in [0, G) with group_ptr[g] <= r
// (group_ptr ascends from 0).  The whole wave searches at once -- lane l
// compares entry base + l, the ballot counts the entries <= r -- so the
// answer costs one load round trip per 64 groups instead of a chain of
// log2(G) dependent loads.  Every lane of the wave must be active; the result
// lies in [0, G) whatever group_ptr holds.
__device__ __forceinline__ int wave_find_group(const int32_t *group_ptr, int G, int r) {
    const int lane = threadIdx.x & 63;
    for (int base = 0;; base += 64) {
        const int g = base + lane;
        const bool le = g < G && group_ptr[g] <= r;
        const int cnt = __popcll(__builtin_amdgcn_ballot_w64(le));
        if (cnt < 64 || base + 64 >= G) return base + cnt > 0 ? base + cnt - 1 : 0;
    }
}

// Wave-wide reductions (wave64) ------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Launch-side status helper.
static inline int hip_status(hipError_t e) { return e == hipSuccess ? SGL_OK : SGL_ERR_HIP; }

// Partial softmax state layout written by split kernels and read by the merge:
//   o part  [B][S][Hq][D] fp32: sum_j exp(s_j - m) v_j  (not normalised)
//   ml part [B][S][Hq][2] fp32: (m, l) with m in log2 units of the scaled
//            score (m = max_j s_j * scale * log2 e), l = sum_j 2^(s_j*scale*log2e - m).
// An empty key set is stored as (m = -inf, l = 0, o = 0).
// Query rows (new token x query head of one KV head) per workgroup of the
// bf16 prefill kernel; the merge of its key splits bounds tiles the same way.
constexpr int kExtendTileRows = 128;

struct PartialBuf {
    float *o;
    float *ml;
    int32_t S;  // split capacity per request
};

// Kernel launchers implemented in the .hip files ----------------------------
int launch_build_req_to_token(int32_t *r2t, int64_t num_rows, int64_t row_stride,
                              const int32_t *req_rows, int32_t batch, const int32_t *prefix_slots,
                              const int64_t *prefix_off, const int32_t *new_slots,
                              const int64_t *new_off, const int32_t *new_col0, hipStream_t st);

int launch_count_bad_slots(const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                           uint32_t *count, hipStream_t st);

// Cascade: lo[r] = the group prefix length of request r clamped to [0,
// seq_lens[r]] -- where its suffix starts -- for r in [0, batch).
struct SuffixStartArgs {
    const int32_t *group_ptr;
    const int32_t *group_prefix_len;
    const int32_t *seq_lens;
    int32_t G, batch;
    int32_t *lo;
    // Optional: the plan of a balanced suffix stage (launch_cascade_balanced),
    // by one more workgroup of the launch that writes lo, from the same group
    // arrays: plan[r] = suffix keys of the requests before r (r <= batch),
    // plan[batch + 1] = keys per run of plan_wgs runs.  A request's suffix is
    // [lo, min(seq_lens, row_stride)), empty if its row is outside the table.
    int64_t *plan;
    int32_t plan_wgs;
    const int32_t *req_rows;
    int64_t num_rows, row_stride;
};
int launch_suffix_start(const SuffixStartArgs &a, hipStream_t st);

// The decode store as a job for the workgroups of some launch: token i of
// n_tokens (row i of k_new / v_new) goes to the slot at position lens[i] - 1
// of table row req_rows[i]; with fp8 set the rows are quantised to e4m3fn
// codes from elt-byte inputs with the per-KV-head factors.  ss.lo, when set,
// also receives the suffix starts.  n_wg: workgroups the carrying launch gives
// the job (decode_store_wgs).
struct DecodeStoreArgs {
    const char *k_new, *v_new;
    uint4 *k_pool, *v_pool;
    int64_t num_slots;
    int32_t row_chunks;     // 16-byte chunks of a pool row
    int32_t head_chunks;    // fp8: 16-byte chunks of one head's codes
    const float *k_scale, *v_scale;
    const int32_t *r2t;
    int64_t num_rows, stride;
    const int32_t *req_rows, *lens;
    int64_t n_tokens;
    int32_t elt;            // input bytes per element (2 bf16, 4 fp32)
    int32_t fp8;
    int32_t n_wg;
    SuffixStartArgs ss;
};
DecodeStoreArgs decode_store_args(int elt, bool fp8, const void *k_new, const void *v_new, int64_t n_tokens,
                                  void *k_pool, void *v_pool, int64_t num_slots, int32_t Hkv, int32_t D,
                                  const float *k_scale, const float *v_scale, const int32_t *r2t,
                                  int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                                  const int32_t *lens, const SuffixStartArgs *ss);
// Workgroups of `threads` threads for the job: about four chunks per thread,
// at most 256, a multiple of 8 (so workgroups numbered after them in the
// same grid keep the XCD they would have without them); 0 for no tokens and
// no suffix starts.
int32_t decode_store_wgs(const DecodeStoreArgs &d, int threads);

// mode 0: slots[i];  mode 1: extend (r2t at prefix_lens[r] + i);  mode 2: decode (r2t at seq_lens[r]-1).
// Mode 2 also writes the suffix starts of *ss when ss is not null (one launch for both).
int launch_store_kv(int mode, int elt, const void *k_new, const void *v_new, int64_t n_tokens,
                    const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                    int32_t Hkv, int32_t D, const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                    const int32_t *req_rows, const int32_t *lens, const int64_t *q_off,
                    int32_t batch, int32_t max_extend_len, hipStream_t st, const SuffixStartArgs *ss = nullptr);

// The same three modes, quantising to e4m3fn codes with per-KV-head factors.
int launch_store_kv_fp8(int mode, int elt, const void *k_new, const void *v_new, int64_t n_tokens,
                        const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                        int32_t Hkv, int32_t D, const float *k_scale, const float *v_scale,
                        const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                        const int32_t *req_rows, const int32_t *lens, const int64_t *q_off,
                        int32_t batch, int32_t max_extend_len, hipStream_t st, const SuffixStartArgs *ss = nullptr);

int launch_extend_f32(const float *q, const float *k_pool, const float *v_pool, int64_t num_slots,
                      const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                      const int32_t *req_rows, const int32_t *prefix_lens, const int64_t *q_off,
                      int32_t batch, int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D,
                      float scale, float *o, float *lse, hipStream_t st);

int launch_extend_bf16(const __bf16 *q, const __bf16 *k_pool, const __bf16 *v_pool,
                       int64_t num_slots, const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                       const int32_t *req_rows, const int32_t *prefix_lens, const int64_t *q_off,
                       int32_t batch, int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D,
                       float scale, __bf16 *o, float *lse, int32_t n_split, int32_t ksplit, PartialBuf part,
                       hipStream_t st);

// Which key range a split kernel covers:
//   kind 0 (flat):   per request r, keys [0, seq_lens[r])
//   kind 1 (prefix): per group g, keys [0, group_prefix_len[g]) of the group's first row,
//                    query rows = every member of the group
//   kind 2 (suffix): per request r, keys [group_prefix_len[group(r)], seq_lens[r])
//   kind 4 (small-q extend): per request r with P = prefix_lens[r] cached keys and
//                    E = q_off[r+1] - q_off[r] new tokens, keys [0, P + E) cut into
//                    n_spl splits of verify_chunk(P + E, n_spl) keys; query rows =
//                    (new token i, q head), row of token i sees keys <= P + i; split
//                    states are indexed by token (q_off[r] + i) instead of request
struct SplitArgs {
    int kind;
    const void *q;
    const void *k_pool;
    const void *v_pool;
    int64_t num_slots;
    const int32_t *r2t;
    int64_t num_rows;
    int64_t row_stride;
    const int32_t *req_rows;
    const int32_t *seq_lens;
    const int32_t *group_ptr;
    const int32_t *group_prefix_len;
    int32_t batch;
    int32_t G;
    int32_t n_sets;        // grid extent over requests (kind 0/2) or groups (kind 1)
    int32_t max_splits;    // grid extent over splits
    int32_t chunk;         // keys per split
    int32_t max_members;   // kind 1: rows of a group = members * (Hq/Hkv)
    int32_t row_blocks;    // kind 1: waves per group (64 rows each) -- set by the launcher
    int32_t Hq, Hkv, D;
    float scale;
    const float *k_scale;  // FP8 KV only: per KV head factors of the K and V codes
    const float *v_scale;
    int32_t xcd_block;     // launch_split_rows: consecutive requests per XCD block
    const int64_t *q_off;          // kind 4: token offsets [batch + 1]
    const int32_t *prefix_lens;    // kind 4: cached keys per request
    int32_t n_spl;                 // kind 4: splits per request
    const int32_t *suffix_lo;      // kind 2, optional: first suffix key of each request
                                   // (launch_suffix_start); else found from the group arrays
    int32_t rounds;                // launch_split_rows, kind 2 with suffix_lo: split rounds in the
                                   // grid (0: all max_splits); each workgroup then also runs the
                                   // non-empty items of the later rounds that share its id modulo
                                   // the grid
    PartialBuf part;
    // Balanced suffix stage (launch_cascade_balanced): plan[r] = first
    // suffix key of request r in the concatenation of all requests' suffixes
    // (r <= batch; plan[batch] = their total), plan[batch + 1] = keys per
    // workgroup; sk_wgs workgroups per head group
    const int64_t *sk_plan;
    int32_t sk_wgs;
    DecodeStoreArgs store;         // kind 1 (launch_split_bf16 / _fp8), optional: a decode
                                   // store run by leading workgroups of the launch
};

int launch_cascade_balanced(const SplitArgs &pa, const SplitArgs &sa, bool fp8, hipStream_t st);

// Keys per split of a small-q extend request with L keys cut into n_spl
// splits (whole 16-key tiles); the split kernel and the merge both use it.
__host__ __device__ __forceinline__ int64_t verify_chunk(int64_t L, int32_t n_spl) {
    const int64_t c = ceil_div64(ceil_div64(L, n_spl), 16) * 16;
    return c < 16 ? 16 : c;
}

int launch_split_f32(const SplitArgs &a, hipStream_t st);
int launch_split_bf16(const SplitArgs &a, hipStream_t st);
int launch_split_fp8(const SplitArgs &a, hipStream_t st);
// kinds 0 and 2 with one workgroup per (request, split) over all KV heads;
// SGL_ERR_UNSUPPORTED for shapes left to the per-head kernels
int launch_split_rows(const SplitArgs &a, bool fp8, hipStream_t st);
// the cascade's prefix (kind 1) and suffix (kind 2) stages in one launch, for
// D = 128 and Hkv a multiple of 4 (at most 16, Hq/Hkv <= 16); the suffix
// uses the whole-row items of launch_split_rows, the prefix four-wave items
// of up to 64 query rows.  Suffix split rounds [0, head_rounds) are
// dispatched before the prefix items, the remaining rounds after them.
// SGL_ERR_UNSUPPORTED for other shapes.
int launch_cascade_split(const SplitArgs &pa, const SplitArgs &sa, int32_t head_rounds, bool fp8, hipStream_t st);
// kinds 0-2 over a latent (MLA) cache: Hkv = 1, 576 score dims, 512 value dims
int launch_split_mla(const SplitArgs &a, hipStream_t st);

// Merge partial states of (optionally) a prefix buffer and a suffix buffer.
//   kind 0: parts = flat splits of r;  kind 3: parts = prefix splits of group(r) for r
//   + suffix splits of r;  kind 4: r is a token of a small-q extend (batch = tokens),
//   parts = the splits of its request (n_req requests, q_off, prefix_lens, n_spl);
//   kind 5: r is a token of a key-split prefill extend (batch = tokens), parts =
//   the chunk_flat-key splits of its query tile's keys (n_req, q_off,
//   prefix_lens, Hkv, row_stride).
struct MergeArgs {
    int kind;
    PartialBuf flat_or_suffix;
    PartialBuf prefix;
    const int32_t *seq_lens;
    const int32_t *group_ptr;
    const int32_t *group_prefix_len;
    int32_t batch, G, chunk_flat, chunk_prefix;
    int32_t Hq, D;
    int out_bf16;
    void *o;
    float *lse;
    const int64_t *q_off;
    const int32_t *prefix_lens;
    int32_t n_req, n_spl;
    int32_t Hkv;           // kind 5: query rows of a tile follow from Hq / Hkv
    int64_t row_stride;    // kind 5: bound on a context (keys past it are not read)
    const int32_t *suffix_lo;   // kind 3, optional: as SplitArgs::suffix_lo
    const int64_t *sk_plan;     // kind 3, optional: suffix states of a balanced suffix stage (SplitArgs::sk_plan)
};

// Balanced suffix stage: the piece of request r that workgroup w takes (its
// run's part inside r) leaves its states in row r + w of the suffix buffer.
// Runs and requests both follow the concatenated suffixes, so of two pieces
// the later one has the larger r or the larger w and never a smaller one:
// the rows are distinct, and below batch + workgroups.
__host__ __device__ __forceinline__ int64_t sk_state_rows(int64_t batch, int64_t wgs) { return batch + wgs; }
int launch_merge(const MergeArgs &a, hipStream_t st);

// Row moves between a page-locked host tier and the pool (kernels_hicache.hip).
// Row move i pairs host row host_rows[i] with pool slot slots[i]; tensor t
// (0 = K, 1 = V; n_t = 1 for a single latent pool) moves row_bytes bytes
// (cpr = row_bytes / 16 chunks of 16 bytes).  dir 0: host -> pool, dir 1:
// pool -> host.  src/dst hold the host tier's device-visible addresses.
struct MoveArgs {
    const char *src[2];
    char *dst[2];
    const int64_t *host_rows;
    const int32_t *slots;
    int64_t n, n_host_rows, num_slots, row_bytes, cpr;
    int n_t;
};
int launch_move_rows(int dir, const MoveArgs &a, hipStream_t st);
