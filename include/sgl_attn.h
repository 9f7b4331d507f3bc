/*
 * sgl_attn.h -- C ABI of the paged prefix-shared attention library for
 * MI355X (gfx950).
 *
 * The library holds the data-parallel hot path behind prefix-shared
 * ("radix") attention: attention over a token-granular paged KV pool whose
 * rows are found through a req_to_token table that a longest-prefix match on
 * a radix tree fills, so a cached shared prefix is read rather than
 * recomputed.  The operations follow the statement of the problem on the
 * pages:
 *   - "SGLang 深度解读" (luoboask.github.io), module 5 "Attention 层 --
 *     RadixAttention 实现": store the current K/V at the slots given by
 *     req_to_token, then run paged attention over the pool;
 *   - "SGLang 深度拆解" (chenxutan.com) section 3.2: the PagedPrefill and
 *     PagedDecode kernels take Q, the paged K/V caches, a page table,
 *     context lengths and cached-prefix lengths;
 *   - the same page, section 2.3: match_prefix / insert / evict / pin on the
 *     radix tree, with reference counts and LRU stamps per node.
 *
 * Conventions for every call
 *   - Plain C types only.  "device" pointers point to GPU memory (any HIP
 *     allocation, e.g. a torch tensor's data_ptr); "host" pointers to CPU
 *     memory.  Streams are hipStream_t passed as void* (NULL = the default
 *     stream).
 *   - The caller owns all device memory: Q/K/V, the pools, req_to_token,
 *     outputs and workspaces.  The library allocates no device memory and
 *     keeps no pointer after a call returns.  Host objects (sgl_kv_pool,
 *     sgl_radix) belong to their handle until *_destroy.
 *   - Device operations only enqueue work on the given stream and return;
 *     their results are ready when the stream is.  Host operations are
 *     synchronous and not thread-safe on one handle.
 *   - Every call returns an sgl_status; no C++ exception crosses the ABI.
 *     Argument checks run before any GPU work is enqueued; a failed call
 *     enqueues nothing.
 *   - Layouts are row-major and dense:  Q/O [tokens, Hq, D];  new K/V
 *     [tokens, Hkv, D];  pools [num_slots, Hkv, D];  req_to_token
 *     [num_rows, row_stride] int32 slot ids;  LSE [tokens, Hq] float32.
 *   - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention with
 *     contiguous groups).  Key j is visible to a query at absolute position
 *     t iff j <= t: the whole cached prefix and the new tokens up to and
 *     including itself.
 *   - Supported: dtype SGL_F32 or SGL_BF16 (outputs in the input dtype,
 *     arithmetic accumulates in fp32), D in {64, 128}, Hq / Hkv in
 *     {1, 2, 4, 8}, Hkv <= 16.  Anything else -> SGL_ERR_UNSUPPORTED.
 *   - Index safety: device kernels never access memory outside the arrays
 *     the arguments describe.  A slot id outside [0, num_slots) read from
 *     req_to_token is replaced by slot 0 (its result is then meaningless but
 *     no fault occurs); sgl_count_bad_slots counts such ids on the device,
 *     stream-ordered.  With the environment variable SGL_ATTN_VALIDATE=1
 *     the device calls first copy the index metadata to the host (a
 *     synchronising step), check it, and return SGL_ERR_INVALID on any
 *     out-of-range slot, row or length, enqueuing nothing; sgl_set_validate
 *     switches this at run time.
 */
#ifndef SGL_ATTN_H
#define SGL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SGL_OK = 0,
    SGL_ERR_INVALID = 1,      /* bad shape, length, index, handle or pointer */
    SGL_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype, D, group size) */
    SGL_ERR_OOM = 3,          /* slot pool exhausted; the pool is unchanged */
    SGL_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
    SGL_ERR_WORKSPACE = 5     /* workspace missing or smaller than required */
} sgl_status;

typedef enum { SGL_F32 = 0, SGL_BF16 = 1 } sgl_dtype;

typedef struct sgl_kv_pool sgl_kv_pool;
typedef struct sgl_radix sgl_radix;

/* Human-readable name of a status code (static string, never NULL). */
const char *sgl_status_string(int status);

/* ABI version of this header (bumped on any signature change). */
int sgl_abi_version(void);

/* Validation of index metadata by the device calls, switchable at run time
 * (process-wide, for every thread):  mode 1 = on, 0 = off, -1 = follow the
 * environment variable SGL_ATTN_VALIDATE (the initial state; "1" = on).
 * With validation on, every device call first copies its index metadata
 * (req_to_token, rows, lengths, offsets, group arrays, slot lists) to the
 * host -- a synchronising step -- and returns SGL_ERR_INVALID, enqueuing
 * nothing, on an out-of-range slot, row, length or offset, a length beyond
 * row_stride or the call's max bound, or (cascade calls) a group whose
 * requests do not share the group's prefix slots.  Returns the previous
 * mode, or -2 (nothing changed) for a mode outside {-1, 0, 1}. */
int sgl_set_validate(int mode);

/* ------------------------------------------------------------------------
 * KV slot pool (host).  The pool shares one set of slots between the prefix
 * cache and running requests ("SGLang：从前端 DSL 到 SRT 服务运行时"
 * (oripoin.cn), section "用基数树实现前缀复用", third bullet).  A page is
 * page_size consecutive slots page*page_size .. +page_size-1 (pages of one
 * or more tokens, same section; vLLM's 16-token pages, chenxutan.com section
 * 2.2).  The free list is FIFO: alloc pops whole pages from its head, free
 * appends them to its tail.
 * ---------------------------------------------------------------------- */

/* num_slots: multiple of page_size, 1 <= page_size <= 1024, num_slots < 2^31.
 * init_order: host [num_slots / page_size] permutation of the page ids giving
 * the initial free-list order, or NULL for 0, 1, 2, ...  (copied).
 * *out receives the handle.  INVALID if init_order is not a permutation. */
int sgl_kv_pool_create(int64_t num_slots, int32_t page_size, const int32_t *init_order,
                       sgl_kv_pool **out);
int sgl_kv_pool_destroy(sgl_kv_pool *pool);

/* Allocate n slots for a request that already holds cur_len tokens whose last
 * slot is last_slot (ignored when cur_len % page_size == 0).  With
 * page_size > 1 the rest of last_slot's page is used first, then whole pages
 * are popped from the free list; the unused tail of the last page stays with
 * the request.  out_slots: host [n].  OOM (pool unchanged) if not enough
 * pages are free. */
int sgl_kv_pool_alloc(sgl_kv_pool *pool, int64_t cur_len, int32_t last_slot, int64_t n,
                      int32_t *out_slots);

/* Return slots to the pool: every slot in host slots[n] that starts a page
 * (slot % page_size == 0) returns its page, in array order.  Other slots are
 * skipped (they belong to a page whose first slot is in the list).  INVALID
 * (pool unchanged) on an out-of-range slot or a page that is already free. */
int sgl_kv_pool_free(sgl_kv_pool *pool, const int32_t *slots, int64_t n);

/* Number of free slots (free pages * page_size), or -1 for a NULL pool. */
int64_t sgl_kv_pool_available(const sgl_kv_pool *pool);

/* ------------------------------------------------------------------------
 * Prefix cache: a compressed radix tree over token ids whose nodes hold the
 * slots of their tokens, a reference count and an LRU stamp
 * (chenxutan.com section 2.3; bhfrc.com news 45689 section 3.1).  Sharing is
 * in whole pages.  A logical clock ticks once per match and once per insert
 * and stamps every node on the path.  Node handles are opaque non-zero ids
 * (0 = the root, i.e. an empty match); a handle stays valid while its node
 * is locked, and until the next evict otherwise.
 * ---------------------------------------------------------------------- */
int sgl_radix_create(int32_t page_size, sgl_radix **out);
int sgl_radix_destroy(sgl_radix *tree);

/* Longest cached prefix of host tokens[n], in whole pages.  *out_len gets its
 * length; out_slots (host, capacity n, may be NULL) gets its slots; *out_node
 * (may be NULL) gets the handle of the node that ends the prefix. */
int sgl_radix_match(sgl_radix *tree, const int32_t *tokens, int64_t n, int32_t *out_slots,
                    int64_t *out_len, uint64_t *out_node);

/* Insert the first floor(n / page_size) pages of host tokens[n] with their
 * host slots[n].  Pages already cached keep the tree's slots; a caller page
 * whose first slot differs from the cached one is a duplicate and is freed
 * to `pool` (may be NULL only if no duplicate can occur), in position order.
 * *out_cached_len (may be NULL) gets how many tokens were already cached.
 * Within a page the slots must be page*page_size + 0, 1, ... (INVALID
 * otherwise, tree unchanged). */
int sgl_radix_insert(sgl_radix *tree, const int32_t *tokens, const int32_t *slots, int64_t n,
                     sgl_kv_pool *pool, int64_t *out_cached_len);

/* Add delta (+1 or -1) to the reference count of every node on the path
 * root..node (pin a prefix / release it, chenxutan.com section 2.3
 * pin_prefix; bhfrc.com news 45689 section 3.2).  INVALID if the handle is
 * unknown or a count would go negative (tree unchanged). */
int sgl_radix_lock(sgl_radix *tree, uint64_t node, int32_t delta);

/* Free at least n_tokens cached tokens if possible: repeatedly remove the
 * last page of the unreferenced leaf with the oldest stamp, returning its
 * page to `pool`, until enough is freed or no unreferenced leaf is left
 * (leaf-first LRU guarded by reference counts, oripoin.cn section
 * "用基数树实现前缀复用").  *out_freed gets the number of tokens freed. */
int sgl_radix_evict(sgl_radix *tree, int64_t n_tokens, sgl_kv_pool *pool, int64_t *out_freed);

/* Cached tokens, and how many of them are unreferenced (evictable). */
int sgl_radix_stats(const sgl_radix *tree, int64_t *out_cached, int64_t *out_evictable);

/* ------------------------------------------------------------------------
 * Batched host bookkeeping: one call per scheduling batch (the scheduler
 * admits, allocates, inserts and releases whole batches -- "SGLang 深度解读"
 * module 2 scheduler loop).  Each is exactly the single-request call applied
 * to requests 0, 1, ..., batch-1 in order; variable-length per-request data
 * is passed as CSR: request r's tokens are tokens[off[r] .. off[r+1]).
 * ---------------------------------------------------------------------- */

/* sgl_radix_match for every request.  Request r's matched slots go to
 * out_slots[off[r] ..] (capacity off[batch]), its length to out_len[r], its
 * node to out_node[r] (may be NULL).  lock != 0 also adds 1 to the reference
 * counts along each matched path (sgl_radix_lock(+1) right after its match). */
int sgl_radix_match_batch(sgl_radix *tree, const int32_t *tokens, const int64_t *off, int32_t batch,
                          int32_t lock, int32_t *out_slots, int64_t *out_len, uint64_t *out_node);

/* sgl_radix_insert for every request: tokens / slots in CSR (same off).
 * out_cached_len: [batch] or NULL.  Stops at the first failing request and
 * returns its status (earlier requests stay inserted). */
int sgl_radix_insert_batch(sgl_radix *tree, const int32_t *tokens, const int32_t *slots,
                           const int64_t *off, int32_t batch, sgl_kv_pool *pool,
                           int64_t *out_cached_len);

/* sgl_radix_lock(node[r], delta) for every request.  All handles are checked
 * first; on error nothing changes. */
int sgl_radix_lock_batch(sgl_radix *tree, const uint64_t *nodes, int32_t batch, int32_t delta);

/* sgl_kv_pool_alloc for every request (cur_len[r], last_slot[r], n[r]);
 * request r's slots go to out_slots[o_r ..] where o_r = n[0] + ... + n[r-1].
 * All or nothing: every request's arguments are checked before any page is
 * popped; if one is invalid (e.g. a last_slot that cannot end a request of
 * cur_len tokens) the call returns SGL_ERR_INVALID, and if the pool cannot
 * serve the whole batch it returns SGL_ERR_OOM; either way the pool is
 * unchanged and out_slots unwritten. */
int sgl_kv_pool_alloc_batch(sgl_kv_pool *pool, const int64_t *cur_len, const int32_t *last_slot,
                            const int64_t *n, int32_t batch, int32_t *out_slots);

/* ------------------------------------------------------------------------
 * Device operations.
 * ---------------------------------------------------------------------- */

/* Build req_to_token rows (GPU scatter).  For request r (0 <= r < batch) the
 * table row req_rows[r] receives, from column new_col0[r] (or, if new_col0 is
 * NULL, from column P_r), the slots new_slots[new_off[r] .. new_off[r+1]),
 * and columns [0, P_r) receive prefix_slots[prefix_off[r] .. prefix_off[r+1])
 * where P_r = prefix_off[r+1] - prefix_off[r].  prefix_slots / prefix_off
 * may both be NULL (P_r = 0, columns outside the new range untouched; this
 * is the decode append).  All arrays are device arrays; offsets are int64
 * CSR offsets starting at 0.  Writes that would fall outside
 * [0, num_rows) x [0, row_stride) are dropped by the kernel. */
int sgl_build_req_to_token(int32_t *r2t, int64_t num_rows, int64_t row_stride,
                           const int32_t *req_rows, int32_t batch,
                           const int32_t *prefix_slots, const int64_t *prefix_off,
                           const int32_t *new_slots, const int64_t *new_off,
                           const int32_t *new_col0, void *stream);

/* Device-side index check, stream-ordered (no host round trip, unlike the
 * validation switch): adds to *count (a device uint32 that the caller zeroes
 * beforehand) the number of slot ids req_to_token[req_rows[r], j],
 * 0 <= j < seq_lens[r], that lie outside [0, num_slots), plus one for every
 * request whose row lies outside [0, num_rows) or whose length lies outside
 * [0, min(row_stride, max_seq_len)].  These are exactly the ids the
 * attention calls would replace by slot 0 (see "Index safety" above); the
 * rows a call reads are the request's first seq_lens[r] columns (for an
 * extend call, prefix_lens[r] plus its new tokens).  All arrays are device
 * arrays; the count is read and written by one vector atomic per wave, so
 * several checks may add to one counter.  The pages say nothing of malformed
 * tables: this is a safety aid for callers that build their own
 * req_to_token, not part of the method. */
int sgl_count_bad_slots(const int32_t *r2t, int64_t num_rows, int64_t row_stride, const int32_t *req_rows,
                        const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                        uint32_t *count, void *stream);

/* Store K/V rows into the pools: token i's K row (Hkv*D elements) goes to
 * k_pool[slots[i]], likewise V ("token_to_kv_pool.write(cache_loc, k, v)",
 * luoboask.github.io module 5).  slots: device [n_tokens]; out-of-range slots
 * are skipped. */
int sgl_store_kv(int dtype, const void *k_new, const void *v_new, int64_t n_tokens,
                 const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                 int32_t Hkv, int32_t D, void *stream);

/* Extend (prefix-aware prefill) attention, chenxutan.com section 3.2
 * PagedPrefill and luoboask.github.io module 5.  Request r has a cached
 * prefix of P_r = prefix_lens[r] tokens and E_r = q_off[r+1] - q_off[r] new
 * tokens; its new token i sits at absolute position P_r + i and is query row
 * q_off[r] + i.  Its K/V row at position j is slot
 * r2t[req_rows[r] * row_stride + j].
 *   q: device [n_tokens, Hq, D];  o: device [n_tokens, Hq, D] (dtype).
 *   k_new / v_new: device [n_tokens, Hkv, D] to be stored first at the slots
 *     of positions P_r .. P_r+E_r-1, or both NULL if already stored.
 *   prefix_lens, req_rows: device int32 [batch];  q_off: device int64
 *     [batch+1], q_off[0] = 0, q_off[batch] = n_tokens.
 *   max_extend_len: host bound >= every E_r (sizes the grid);
 *   lse: device float32 [n_tokens, Hq] log-sum-exp of the scaled scores
 *     (natural log), or NULL.
 *   workspace: device scratch of sgl_extend_workspace_size(...) bytes (may be
 *     NULL when that size is 0), given the same batch, n_tokens,
 *     max_extend_len, row_stride and heads as the call.  The size is non-zero
 *     (a) for max_extend_len * (Hq / Hkv) <= 16 -- a few new tokens per
 *     request, as in the verify step of speculative decoding -- which runs as
 *     a split-K pass over each request's keys plus a log-sum-exp merge, and
 *     (b) when the prefill grid (one workgroup per request, 128 query rows and
 *     KV head) is small and row_stride allows long contexts, where each
 *     workgroup's keys are split in 4096-key multiples and merged the same way.
 *     Either way the result is the same attention (bf16 calls; fp32 calls
 *     ignore the workspace).  A smaller workspace, or none, is accepted: the
 *     call then runs the prefill kernel without splits (the same attention
 *     within rounding, only slower), so a workspace sized for other bounds
 *     never makes the call fail.
 * scale multiplies q.k (normally 1/sqrt(D)). */
int sgl_extend_attn(int dtype, const void *q, const void *k_new, const void *v_new,
                    void *k_pool, void *v_pool, int64_t num_slots,
                    const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                    const int32_t *req_rows, const int32_t *prefix_lens, const int64_t *q_off,
                    int32_t batch, int64_t n_tokens, int32_t max_extend_len,
                    int32_t Hq, int32_t Hkv, int32_t D, float scale,
                    void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream);
size_t sgl_extend_workspace_size(int32_t batch, int64_t n_tokens, int32_t max_extend_len,
                                 int64_t row_stride, int32_t Hq, int32_t Hkv, int32_t D);

/* Decode attention: one query token per request over its whole context,
 * chenxutan.com section 3.2 PagedDecode.  seq_lens[r] (device int32)
 * INCLUDES the current token, whose K/V sits at position seq_lens[r]-1
 * (stored first from k_new / v_new [batch, Hkv, D] when they are not NULL).
 *   q, o: device [batch, Hq, D];  lse: device float32 [batch, Hq] or NULL.
 *   max_seq_len: host bound >= every seq_lens[r] (sizes the split-K grid).
 *   workspace: sgl_decode_workspace_size(...) bytes. */
int sgl_decode_attn(int dtype, const void *q, const void *k_new, const void *v_new,
                    void *k_pool, void *v_pool, int64_t num_slots,
                    const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                    const int32_t *req_rows, const int32_t *seq_lens,
                    int32_t batch, int32_t max_seq_len,
                    int32_t Hq, int32_t Hkv, int32_t D, float scale,
                    void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream);
size_t sgl_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t Hq, int32_t Hkv,
                                 int32_t D);

/* Cascade decode: as sgl_decode_attn, but the requests form G groups that
 * share a cached prefix (sibling requests of one radix subtree: parallel
 * samples of one prompt, bhfrc.com news 45689 section 1.3).  Requests
 * group_ptr[g] .. group_ptr[g+1]-1 form group g (group_ptr: device int32
 * [G+1], group_ptr[0] = 0, group_ptr[G] = batch) and share their first
 * group_prefix_len[g] (device int32 [G]) KV positions.  The shared prefix is
 * read ONCE per group for all its requests' queries, each request's own
 * suffix is read per request, and the two partial softmax states are merged
 * with the log-sum-exp rule.  The result equals sgl_decode_attn.
 * Precondition: within a group all req_to_token rows hold the same slots in
 * columns [0, group_prefix_len[g]) (the prefix slots are read from the row
 * of the group's first request) and group_prefix_len[g] <= seq_lens[r] for
 * its requests; when the call stores the current token (k_new given), the
 * prefix ends before it: group_prefix_len[g] < seq_lens[r], and the slot of
 * position seq_lens[r]-1 is none of the group's prefix slots (the store may
 * run while the prefix is being read).  Validation mode returns
 * SGL_ERR_INVALID for a call that breaks either.
 * max_group_size, max_prefix_len: host bounds (grid sizing);
 * max_group_size * (Hq / Hkv) <= 4096.  Up to 64 query rows of a group
 * (request x query head) share one read of the prefix; larger groups read it
 * once per 64 rows.
 * workspace: sgl_cascade_workspace_size(...) bytes (both stages' split states
 * and each request's suffix start, written by the call before it reads them). */
int sgl_cascade_decode_attn(int dtype, const void *q, const void *k_new, const void *v_new,
                            void *k_pool, void *v_pool, int64_t num_slots,
                            const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                            const int32_t *req_rows, const int32_t *seq_lens,
                            const int32_t *group_ptr, const int32_t *group_prefix_len,
                            int32_t batch, int32_t G, int32_t max_seq_len,
                            int32_t max_group_size, int32_t max_prefix_len,
                            int32_t Hq, int32_t Hkv, int32_t D, float scale,
                            void *o, float *lse, void *workspace, size_t workspace_bytes,
                            void *stream);
size_t sgl_cascade_workspace_size(int32_t batch, int32_t G, int32_t max_seq_len,
                                  int32_t max_group_size, int32_t max_prefix_len,
                                  int32_t Hq, int32_t Hkv, int32_t D);

/* Allocation-free cascade decode, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid allocation.  Same arguments, semantics and
 * result as sgl_cascade_decode_attn, without the workspace: the split states
 * (and the requests' suffix starts) live in a static device array of
 * sgl_static_scratch_bytes() = 128 MiB that every GPU the library runs on
 * holds from its first use until the process ends.  The call allocates no device memory (and calls no allocating
 * library routine); with validation on (sgl_set_validate) it still copies
 * the index metadata into host memory first.  A call whose split states do
 * not fit 128 MiB -- the sizing rule of sgl_cascade_workspace_size with the
 * prefix splits doubled up to 512 keys and the suffix splits up to 1024;
 * e.g. 256 requests x 32 query heads x D 128 over contexts up to 8k fit --
 * returns SGL_ERR_WORKSPACE and enqueues
 * nothing.  Every call on one GPU shares that GPU's array, and every state a
 * call reads it has written first, so nothing needs clearing between calls;
 * calls on one stream are ordered, but calls that can overlap on one GPU
 * (several streams, or several host threads) race on the array and must not
 * be issued. */
int sgl_cascade_decode_attn_static(int dtype, const void *q, const void *k_new, const void *v_new,
                                   void *k_pool, void *v_pool, int64_t num_slots,
                                   const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                                   const int32_t *req_rows, const int32_t *seq_lens,
                                   const int32_t *group_ptr, const int32_t *group_prefix_len,
                                   int32_t batch, int32_t G, int32_t max_seq_len,
                                   int32_t max_group_size, int32_t max_prefix_len,
                                   int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                   void *o, float *lse, void *stream);
size_t sgl_static_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * FP8 KV cache.  SGLang can keep the KV cache in FP8, which halves its bytes
 * ("SGLang 深度拆解" (chenxutan.com) section 4.3; "Lecture 16 · 案例研究：SGLang"
 * (semidirectx.com) section 4 "More engineering" lists an FP8 KV cache among
 * the kernel work).  The
 * pages fix neither format nor scaling; this library uses:
 *   - pools of uint8 OCP e4m3fn codes, layout [num_slots, Hkv, D] as for the
 *     bf16 pools (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 *     infinity; S.1111.111 is NaN; largest finite 448);
 *   - one fp32 factor per KV head for K (k_scale[Hkv]) and one for V
 *     (v_scale[Hkv]), device arrays: code c of head kv stands for
 *     value(c) * scale[kv];
 *   - quantisation of x (head kv): y = x / scale[kv] in fp32, clamped to
 *     [-448, 448], rounded to the nearest e4m3fn value, ties to the even
 *     code; the sign is kept (a negative y that rounds to 0 gives 0x80).
 *     A NaN input gives a NaN code.
 * Attention then equals attention over the dequantised K and V.
 * ---------------------------------------------------------------------- */

/* Quantise and store K/V rows: as sgl_store_kv, with k_new / v_new of
 * dtype (SGL_F32 or SGL_BF16, [n_tokens, Hkv, D]) written as codes into the
 * uint8 pools k_pool / v_pool [num_slots, Hkv, D]. */
int sgl_store_kv_fp8(int dtype, const void *k_new, const void *v_new, int64_t n_tokens,
                     const int32_t *slots, void *k_pool, void *v_pool, int64_t num_slots,
                     int32_t Hkv, int32_t D, const float *k_scale, const float *v_scale, void *stream);

/* sgl_decode_attn over an FP8 KV cache.  dtype must be SGL_BF16 (q, o and,
 * when given, k_new / v_new [batch, Hkv, D], which are quantised and stored
 * first); k_pool / v_pool hold codes, k_scale / v_scale their per-head
 * factors.  The workspace is sgl_decode_workspace_size(...) bytes, as for
 * the bf16 call. */
int sgl_decode_attn_fp8kv(int dtype, const void *q, const void *k_new, const void *v_new,
                          void *k_pool, void *v_pool, const float *k_scale, const float *v_scale,
                          int64_t num_slots, const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                          const int32_t *req_rows, const int32_t *seq_lens,
                          int32_t batch, int32_t max_seq_len,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale,
                          void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* sgl_cascade_decode_attn over an FP8 KV cache (arguments as
 * sgl_decode_attn_fp8kv plus the group arguments of sgl_cascade_decode_attn;
 * workspace sgl_cascade_workspace_size(...) bytes).  The result equals
 * sgl_decode_attn_fp8kv. */
int sgl_cascade_decode_attn_fp8kv(int dtype, const void *q, const void *k_new, const void *v_new,
                                  void *k_pool, void *v_pool, const float *k_scale, const float *v_scale,
                                  int64_t num_slots, const int32_t *r2t, int64_t num_rows,
                                  int64_t row_stride, const int32_t *req_rows, const int32_t *seq_lens,
                                  const int32_t *group_ptr, const int32_t *group_prefix_len,
                                  int32_t batch, int32_t G, int32_t max_seq_len,
                                  int32_t max_group_size, int32_t max_prefix_len,
                                  int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                  void *o, float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* ------------------------------------------------------------------------
 * Latent (MLA-style) decode.  With the decompression matrices absorbed into
 * the query and output projections, DeepSeek's MLA attention runs directly on
 * the compressed latent ("Lecture 16 · 案例研究：SGLang" (semidirectx.com)
 * section 4, "More engineering"): each token has ONE latent row of Dqk = 576
 * dims (512 compressed K/V dims followed by 64 RoPE dims) shared by every
 * query head; the score of head h is q_h . latent (all 576 dims) * scale and
 * the value is the latent's first Dv = 512 dims.  It is grouped-query
 * attention with one KV head whose value rows are a prefix of its key rows.
 *   q: device bf16 [batch, Hq, 576], Hq a multiple of 16 up to 128;
 *   kv_pool: device bf16 [num_slots, 576] (the latent of every slot);
 *   kv_new: device bf16 [batch, 576] stored first at position seq_lens[r]-1,
 *     or NULL;
 *   o: device bf16 [batch, Hq, 512];  lse: device float32 [batch, Hq] or NULL;
 *   scale multiplies q . latent (1/sqrt(192) for DeepSeek's 128 + 64 dims).
 * Other arguments as sgl_decode_attn / sgl_cascade_decode_attn (the cascade's
 * precondition on shared prefix slots applies).  Dqk must be 576 and Dv 512
 * (else SGL_ERR_UNSUPPORTED).  Workspace: the sizes below.
 * ---------------------------------------------------------------------- */
int sgl_mla_decode_attn(const void *q, const void *kv_new, void *kv_pool, int64_t num_slots,
                        const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                        const int32_t *req_rows, const int32_t *seq_lens, int32_t batch,
                        int32_t max_seq_len, int32_t Hq, int32_t Dqk, int32_t Dv, float scale,
                        void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream);
size_t sgl_mla_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t Hq, int32_t Dv);
int sgl_mla_cascade_decode_attn(const void *q, const void *kv_new, void *kv_pool, int64_t num_slots,
                                const int32_t *r2t, int64_t num_rows, int64_t row_stride,
                                const int32_t *req_rows, const int32_t *seq_lens,
                                const int32_t *group_ptr, const int32_t *group_prefix_len,
                                int32_t batch, int32_t G, int32_t max_seq_len,
                                int32_t max_group_size, int32_t max_prefix_len,
                                int32_t Hq, int32_t Dqk, int32_t Dv, float scale,
                                void *o, float *lse, void *workspace, size_t workspace_bytes,
                                void *stream);
size_t sgl_mla_cascade_workspace_size(int32_t batch, int32_t G, int32_t max_seq_len,
                                      int32_t max_group_size, int32_t max_prefix_len,
                                      int32_t Hq, int32_t Dv);

/* ----------------------------------------------------------------------
 * Host tier of the KV cache (HiCache).  KV rows that leave the GPU pool are
 * kept in a larger page-locked host-memory tier and brought back into pool
 * slots when a later request matches them ("SGLang：从前端 DSL 到 SRT 服务运行时",
 * section "从 2024 年论文到今天的缓存栈", the HiCache bullet: GPU memory is the
 * first tier, host memory the second; a prefix matched in a lower tier is
 * prefetched, and rows are written back).  The pages give no layout; here a
 * host row has exactly the pool's row layout (Hkv * D elements of the pool's
 * dtype, or one latent row), so both moves copy bytes unchanged.
 *
 *   sgl_hicache_prefetch:   for i < n:  pool[slots[i]] <- host[host_rows[i]]
 *   sgl_hicache_write_back: for i < n:  host[host_rows[i]] <- pool[slots[i]]
 *
 * Each tensor pair (K and V; or only K with host_v = v_pool = NULL for a
 * single latent pool) moves row_bytes bytes per row; row_bytes must be a
 * positive multiple of 16 (bf16 Hkv*D*2, fp8 Hkv*D, latent 576*2).
 *   host_k, host_v: PAGE-LOCKED host memory (hipHostMalloc, or a pinned
 *     torch tensor) of n_host_rows rows; the call checks that the whole
 *     range is page-locked and mapped for the device, else SGL_ERR_INVALID.
 *     The kernel reads or writes it directly over the host link.
 *   k_pool, v_pool: device [num_slots] rows;
 *   host_rows: device int64 [n];  slots: device int32 [n];
 *   all four buffers 16-byte aligned.
 * Destinations must be distinct (slots for a prefetch, host_rows for a
 * write-back); sources may repeat.  A move whose host row or slot lies
 * outside its buffer is skipped (no access is made); with
 * SGL_ATTN_VALIDATE=1 such indices, and repeated destinations, return
 * SGL_ERR_INVALID before anything is launched.  Stream-ordered: the caller
 * synchronises before reading the host tier after a write-back.  n = 0 is a
 * no-op.
 * ---------------------------------------------------------------------- */
int sgl_hicache_prefetch(const void *host_k, const void *host_v, int64_t n_host_rows,
                         const int64_t *host_rows, const int32_t *slots, int64_t n,
                         void *k_pool, void *v_pool, int64_t num_slots, int64_t row_bytes,
                         void *stream);
int sgl_hicache_write_back(const void *k_pool, const void *v_pool, int64_t num_slots,
                           const int32_t *slots, const int64_t *host_rows, int64_t n,
                           void *host_k, void *host_v, int64_t n_host_rows, int64_t row_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SGL_ATTN_H */
