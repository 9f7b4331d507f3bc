// host_cache.cpp -- KV slot pool and prefix cache (compressed radix tree).
//
// Host bookkeeping behind the device path: it decides which pool slots a
// request's tokens use (a cached prefix's slots come from the tree, new
// tokens get fresh slots) and therefore what req_to_token holds.
//
//   * Pool: FIFO free list of pages.  The pool is shared by the cache and the
//     running requests ("SGLang：从前端 DSL 到 SRT 服务运行时" (oripoin.cn),
//     section "用基数树实现前缀复用").
//   * Tree: a compressed radix tree -- every edge holds a run of whole pages
//     (bhfrc.com news 45689 section 3.1: children found by their first token,
//     longest common prefix along the edge, split on divergence).  Each node
//     keeps the slots of its tokens, a reference count and an LRU stamp
//     ("SGLang 深度拆解" (chenxutan.com) section 2.3, the per-node fields).
//
// Semantics that the pages leave open (shared with the test model, which is
// an uncompressed trie):
//   - a logical clock ticks once per match and per insert; every node on the
//     touched path gets the new stamp.  A match or insert that ends inside an
//     edge splits it, so that stamps (and handles) stay exact per page;
//   - a split keeps the original node object as the LOWER part (it still ends
//     where it ended), so outstanding handles keep denoting the same prefix;
//   - eviction removes the last page of the unreferenced leaf with the
//     oldest stamp, one page at a time, freeing pages tail-first.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <functional>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "sgl_attn.h"

// One bit per page: is it on the free list.  A bit vector (128 KiB for 2^20
// pages) stays cache-resident while pages are allocated and freed in random
// order, where a byte per page would miss on nearly every access.
struct PageBits {
    std::vector<uint64_t> w;
    int64_t n = 0;
    void assign(int64_t n_pages) {
        n = n_pages;
        w.assign((size_t)((n_pages + 63) / 64), 0);
    }
    int64_t size() const { return n; }
    bool operator[](int64_t i) const { return (w[(size_t)(i >> 6)] >> (i & 63)) & 1; }
    void set(int64_t i) { w[(size_t)(i >> 6)] |= uint64_t(1) << (i & 63); }
    void clear(int64_t i) { w[(size_t)(i >> 6)] &= ~(uint64_t(1) << (i & 63)); }
};

// FIFO of free page ids in a ring of capacity = pages of the pool (the list
// never holds more).
struct PageRing {
    std::vector<int32_t> buf;
    int64_t head = 0, count = 0;
    void reserve(int64_t n_pages) { buf.assign((size_t)n_pages, 0); }
    int64_t size() const { return count; }
    int32_t front() const { return buf[(size_t)head]; }
    void pop_front() {
        head = head + 1 == (int64_t)buf.size() ? 0 : head + 1;
        count--;
    }
    void push_back(int32_t pg) {
        int64_t tail = head + count;
        if (tail >= (int64_t)buf.size()) tail -= (int64_t)buf.size();
        buf[(size_t)tail] = pg;
        count++;
    }
};

struct sgl_kv_pool {
    int64_t num_slots = 0;
    int32_t page = 1;
    PageRing free_pages;  // head = front
    PageBits is_free;
};

namespace {

struct Node {
    uint64_t id = 0;
    Node *parent = nullptr;
    std::vector<int32_t> tokens;  // edge label, a whole number of pages
    std::vector<int32_t> slots;   // slot of every token on the edge
    std::vector<Node *> children;
    int64_t ref = 0;
    uint64_t stamp = 0;
};

}  // namespace

struct sgl_radix {
    int32_t page = 1;
    uint64_t clock = 0;
    uint64_t next_id = 1;
    Node root;
    std::unordered_map<uint64_t, Node *> by_id;
    ~sgl_radix() {
        std::vector<Node *> stack(root.children.begin(), root.children.end());
        while (!stack.empty()) {
            Node *n = stack.back();
            stack.pop_back();
            stack.insert(stack.end(), n->children.begin(), n->children.end());
            delete n;
        }
    }
};

namespace {

template <class F>
int guarded(F &&f) {
    try {
        return f();
    } catch (const std::bad_alloc &) {
        return SGL_ERR_OOM;
    } catch (...) {
        return SGL_ERR_INVALID;
    }
}

bool page_equal(const int32_t *a, const int32_t *b, int32_t p) {
    return std::memcmp(a, b, sizeof(int32_t) * (size_t)p) == 0;
}

// Child of `n` whose edge starts with the page at `tok`, or null.
Node *find_child(const Node *n, const int32_t *tok, int32_t p) {
    for (Node *c : n->children)
        if (page_equal(c->tokens.data(), tok, p)) return c;
    return nullptr;
}

// Number of whole pages that `c`'s edge shares with tok[0 .. avail_pages*p):
// the first differing token, rounded down to a page.  Long equal runs (a
// cached prefix) are compared with memcmp -- whole range first, then 64-token
// blocks -- and only the block holding the first difference token by token.
int64_t edge_common_pages(const Node *c, const int32_t *tok, int64_t avail_pages, int32_t p) {
    const int64_t edge_pages = (int64_t)c->tokens.size() / p;
    const int64_t lim = std::min(edge_pages, avail_pages) * p;
    const int32_t *e = c->tokens.data();
    if (std::memcmp(e, tok, sizeof(int32_t) * (size_t)lim) == 0) return lim / p;
    constexpr int64_t BLK = 64;
    int64_t i = 0;
    while (i + BLK <= lim && std::memcmp(e + i, tok + i, sizeof(int32_t) * BLK) == 0) i += BLK;
    while (i < lim && e[i] == tok[i]) i++;
    return i / p;
}

// Split `c` after `k` pages: a new upper node takes the first k pages and
// becomes c's parent; c keeps the rest (and its identity).
Node *split(sgl_radix *t, Node *c, int64_t k) {
    const int32_t p = t->page;
    Node *u = new Node();
    u->id = t->next_id++;
    u->parent = c->parent;
    u->tokens.assign(c->tokens.begin(), c->tokens.begin() + k * p);
    u->slots.assign(c->slots.begin(), c->slots.begin() + k * p);
    u->ref = c->ref;
    u->stamp = c->stamp;
    c->tokens.erase(c->tokens.begin(), c->tokens.begin() + k * p);
    c->slots.erase(c->slots.begin(), c->slots.begin() + k * p);
    Node *par = c->parent;
    std::replace(par->children.begin(), par->children.end(), c, u);
    u->children.push_back(c);
    c->parent = u;
    t->by_id[u->id] = u;
    return u;
}

int pool_free_pages(sgl_kv_pool *pool, const std::vector<int32_t> &pages) {
    // Mark pages free one by one; a page that is out of range, already free,
    // or repeated in `pages` fails the call, and the marks made so far are
    // undone, so a failed call leaves the pool unchanged.
    size_t i = 0;
    for (; i < pages.size(); i++) {
        const int32_t pg = pages[i];
        if (pg < 0 || (int64_t)pg >= pool->is_free.size() || pool->is_free[pg]) break;
        pool->is_free.set(pg);
    }
    if (i < pages.size()) {
        for (size_t j = 0; j < i; j++) pool->is_free.clear(pages[j]);
        return SGL_ERR_INVALID;
    }
    for (int32_t pg : pages) pool->free_pages.push_back(pg);
    return SGL_OK;
}

}  // namespace

extern "C" {

const char *sgl_status_string(int status) {
    switch (status) {
        case SGL_OK: return "SGL_OK";
        case SGL_ERR_INVALID: return "SGL_ERR_INVALID";
        case SGL_ERR_UNSUPPORTED: return "SGL_ERR_UNSUPPORTED";
        case SGL_ERR_OOM: return "SGL_ERR_OOM";
        case SGL_ERR_HIP: return "SGL_ERR_HIP";
        case SGL_ERR_WORKSPACE: return "SGL_ERR_WORKSPACE";
        default: return "SGL_ERR_UNKNOWN";
    }
}

int sgl_kv_pool_create(int64_t num_slots, int32_t page_size, const int32_t *init_order,
                       sgl_kv_pool **out) {
    if (!out || page_size < 1 || page_size > 1024 || num_slots < page_size ||
        num_slots % page_size != 0 || num_slots >= ((int64_t)1 << 31))
        return SGL_ERR_INVALID;
    return guarded([&] {
        const int64_t n_pages = num_slots / page_size;
        auto *pool = new sgl_kv_pool();
        pool->num_slots = num_slots;
        pool->page = page_size;
        pool->is_free.assign(n_pages);
        pool->free_pages.reserve(n_pages);
        for (int64_t i = 0; i < n_pages; i++) {
            int32_t pg = init_order ? init_order[i] : (int32_t)i;
            if (pg < 0 || pg >= n_pages || pool->is_free[pg]) {
                delete pool;
                return (int)SGL_ERR_INVALID;
            }
            pool->is_free.set(pg);
            pool->free_pages.push_back(pg);
        }
        *out = pool;
        return (int)SGL_OK;
    });
}

int sgl_kv_pool_destroy(sgl_kv_pool *pool) {
    delete pool;
    return SGL_OK;
}

// Slots of the partly filled last page a request of cur_len tokens (last slot
// last_slot) fills first when it allocates n more, or -1 if last_slot cannot
// be the slot of position cur_len - 1 (out of range, or at the wrong offset
// within its page).
static int64_t partial_fill(const sgl_kv_pool *pool, int64_t cur_len, int32_t last_slot, int64_t n) {
    const int32_t p = pool->page;
    if (p == 1 || cur_len % p == 0) return 0;
    const int64_t fill = std::min<int64_t>(n, p - cur_len % p);
    if (fill > 0 && (last_slot < 0 || (int64_t)last_slot + fill >= pool->num_slots ||
                     (last_slot % p) != (cur_len - 1) % p))
        return -1;
    return fill;
}

int sgl_kv_pool_alloc(sgl_kv_pool *pool, int64_t cur_len, int32_t last_slot, int64_t n,
                      int32_t *out_slots) {
    if (!pool || n < 0 || cur_len < 0 || (n > 0 && !out_slots)) return SGL_ERR_INVALID;
    const int32_t p = pool->page;
    const int64_t fill = partial_fill(pool, cur_len, last_slot, n);
    if (fill < 0) return SGL_ERR_INVALID;
    const int64_t need = (n - fill + p - 1) / p;
    if (need > (int64_t)pool->free_pages.size()) return SGL_ERR_OOM;
    int64_t k = 0;
    for (; k < fill; k++) out_slots[k] = last_slot + 1 + (int32_t)k;
    for (int64_t i = 0; i < need; i++) {
        int32_t pg = pool->free_pages.front();
        pool->free_pages.pop_front();
        pool->is_free.clear(pg);
        for (int32_t j = 0; j < p && k < n; j++) out_slots[k++] = pg * p + j;
    }
    return SGL_OK;
}

int sgl_kv_pool_free(sgl_kv_pool *pool, const int32_t *slots, int64_t n) {
    if (!pool || n < 0 || (n > 0 && !slots)) return SGL_ERR_INVALID;
    return guarded([&] {
        std::vector<int32_t> pages;
        const int32_t p = pool->page;
        pages.reserve((size_t)(p == 1 ? n : n / p + 1));
        for (int64_t i = 0; i < n; i++) {
            int32_t s = slots[i];
            if (s < 0 || s >= pool->num_slots) return (int)SGL_ERR_INVALID;
            if (p == 1) pages.push_back(s);
            else if (s % p == 0) pages.push_back(s / p);
        }
        return pool_free_pages(pool, pages);
    });
}

int64_t sgl_kv_pool_available(const sgl_kv_pool *pool) {
    if (!pool) return -1;
    return (int64_t)pool->free_pages.size() * pool->page;
}

int sgl_radix_create(int32_t page_size, sgl_radix **out) {
    if (!out || page_size < 1 || page_size > 1024) return SGL_ERR_INVALID;
    return guarded([&] {
        auto *t = new sgl_radix();
        t->page = page_size;
        t->root.id = 0;
        *out = t;
        return (int)SGL_OK;
    });
}

int sgl_radix_destroy(sgl_radix *tree) {
    delete tree;
    return SGL_OK;
}

int sgl_radix_match(sgl_radix *t, const int32_t *tokens, int64_t n, int32_t *out_slots,
                    int64_t *out_len, uint64_t *out_node) {
    if (!t || n < 0 || (n > 0 && !tokens)) return SGL_ERR_INVALID;
    return guarded([&] {
        const int32_t p = t->page;
        const uint64_t now = ++t->clock;
        Node *node = &t->root;
        int64_t pos = 0;
        while ((n - pos) / p > 0) {
            Node *c = find_child(node, tokens + pos, p);
            if (!c) break;
            int64_t k = edge_common_pages(c, tokens + pos, (n - pos) / p, p);
            int64_t edge_pages = (int64_t)c->tokens.size() / p;
            if (k < edge_pages) c = split(t, c, k);
            if (out_slots)
                std::memcpy(out_slots + pos, c->slots.data(), sizeof(int32_t) * (size_t)(k * p));
            c->stamp = now;
            pos += k * p;
            node = c;
            if (k < edge_pages) break;
        }
        if (out_len) *out_len = pos;
        if (out_node) *out_node = node->id;
        return (int)SGL_OK;
    });
}

int sgl_radix_insert(sgl_radix *t, const int32_t *tokens, const int32_t *slots, int64_t n,
                     sgl_kv_pool *pool, int64_t *out_cached_len) {
    if (!t || n < 0 || (n > 0 && (!tokens || !slots))) return SGL_ERR_INVALID;
    const int32_t p = t->page;
    const int64_t n_ins = n / p * p;
    if (p == 1) {
        int32_t mn = 0;
        for (int64_t i = 0; i < n_ins; i++) mn = std::min(mn, slots[i]);
        if (mn < 0) return SGL_ERR_INVALID;
    } else {
        for (int64_t i = 0; i < n_ins; i += p) {
            if (slots[i] < 0 || slots[i] % p != 0) return SGL_ERR_INVALID;
            for (int32_t j = 1; j < p; j++)
                if (slots[i + j] != slots[i] + j) return SGL_ERR_INVALID;
        }
    }
    return guarded([&] {
        // Pass 1 (read only): how much is cached and which caller pages are duplicates.
        std::vector<int32_t> dup_pages;
        int64_t cached = 0;
        {
            const Node *node = &t->root;
            int64_t pos = 0;
            while (pos < n_ins) {
                const Node *c = find_child(node, tokens + pos, p);
                if (!c) break;
                int64_t k = edge_common_pages(c, tokens + pos, (n_ins - pos) / p, p);
                // the caller's slots usually are the tree's (they came from a match)
                if (std::memcmp(c->slots.data(), slots + pos, sizeof(int32_t) * (size_t)(k * p)) != 0)
                    for (int64_t i = 0; i < k; i++)
                        if (c->slots[i * p] != slots[pos + i * p]) dup_pages.push_back(slots[pos + i * p] / p);
                pos += k * p;
                if (k < (int64_t)c->tokens.size() / p) break;
                node = c;
            }
            cached = pos;
        }
        if (!dup_pages.empty()) {
            if (!pool || pool->page != p) return (int)SGL_ERR_INVALID;
            for (int32_t pg : dup_pages)
                if (pg < 0 || (int64_t)pg >= pool->is_free.size() || pool->is_free[pg])
                    return (int)SGL_ERR_INVALID;
            std::vector<int32_t> sorted = dup_pages;
            std::sort(sorted.begin(), sorted.end());
            if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
                return (int)SGL_ERR_INVALID;
        }
        // Pass 2: modify.
        const uint64_t now = ++t->clock;
        Node *node = &t->root;
        int64_t pos = 0;
        while (pos < n_ins) {
            Node *c = find_child(node, tokens + pos, p);
            if (!c) break;
            int64_t k = edge_common_pages(c, tokens + pos, (n_ins - pos) / p, p);
            if (k < (int64_t)c->tokens.size() / p) c = split(t, c, k);
            c->stamp = now;
            pos += k * p;
            node = c;
        }
        if (pos < n_ins) {
            Node *leaf = new Node();
            leaf->id = t->next_id++;
            leaf->parent = node;
            leaf->tokens.assign(tokens + pos, tokens + n_ins);
            leaf->slots.assign(slots + pos, slots + n_ins);
            leaf->stamp = now;
            node->children.push_back(leaf);
            t->by_id[leaf->id] = leaf;
        }
        if (!dup_pages.empty()) {
            int rc = pool_free_pages(pool, dup_pages);
            if (rc != SGL_OK) return rc;
        }
        if (out_cached_len) *out_cached_len = cached;
        return (int)SGL_OK;
    });
}

int sgl_radix_lock(sgl_radix *t, uint64_t node_id, int32_t delta) {
    if (!t || (delta != 1 && delta != -1)) return SGL_ERR_INVALID;
    if (node_id == 0) return SGL_OK;  // the root carries no count
    auto it = t->by_id.find(node_id);
    if (it == t->by_id.end()) return SGL_ERR_INVALID;
    for (Node *x = it->second; x && x != &t->root; x = x->parent)
        if (x->ref + delta < 0) return SGL_ERR_INVALID;
    for (Node *x = it->second; x && x != &t->root; x = x->parent) x->ref += delta;
    return SGL_OK;
}

int sgl_radix_evict(sgl_radix *t, int64_t n_tokens, sgl_kv_pool *pool, int64_t *out_freed) {
    if (!t || !pool || pool->page != t->page || n_tokens < 0) return SGL_ERR_INVALID;
    return guarded([&] {
        const int32_t p = t->page;
        using Item = std::pair<uint64_t, Node *>;  // (stamp, node); stamps of leaves are distinct
        std::priority_queue<Item, std::vector<Item>, std::greater<Item>> heap;
        std::vector<Node *> stack(t->root.children.begin(), t->root.children.end());
        while (!stack.empty()) {
            Node *x = stack.back();
            stack.pop_back();
            if (x->children.empty()) {
                if (x->ref == 0) heap.push({x->stamp, x});
            } else {
                stack.insert(stack.end(), x->children.begin(), x->children.end());
            }
        }
        int64_t freed = 0;
        std::vector<int32_t> pages;
        while (freed < n_tokens && !heap.empty()) {
            Node *x = heap.top().second;
            heap.pop();
            // its pages go tail-first: all of them if the leaf goes entirely
            const int64_t take = std::min<int64_t>((int64_t)x->tokens.size() / p, (n_tokens - freed + p - 1) / p);
            const size_t keep = x->tokens.size() - (size_t)take * p;
            for (size_t e = x->tokens.size(); e > keep; e -= p) pages.push_back(p == 1 ? x->slots[e - 1] : x->slots[e - p] / p);
            x->tokens.resize(keep);
            x->slots.resize(keep);
            freed += take * p;
            if (x->tokens.empty()) {
                Node *par = x->parent;
                par->children.erase(std::find(par->children.begin(), par->children.end(), x));
                t->by_id.erase(x->id);
                delete x;
                if (par != &t->root && par->children.empty() && par->ref == 0)
                    heap.push({par->stamp, par});
            }
        }
        // Pages cut from the tree go back to the pool.  A page the pool does not
        // know (slots inserted from another pool) or already holds is skipped.
        for (int32_t pg : pages) {
            if (pg < 0 || (int64_t)pg >= pool->is_free.size() || pool->is_free[pg]) continue;
            pool->is_free.set(pg);
            pool->free_pages.push_back(pg);
        }
        if (out_freed) *out_freed = freed;
        return (int)SGL_OK;
    });
}

int sgl_radix_stats(const sgl_radix *t, int64_t *out_cached, int64_t *out_evictable) {
    if (!t) return SGL_ERR_INVALID;
    int64_t cached = 0, evictable = 0;
    std::vector<const Node *> stack(t->root.children.begin(), t->root.children.end());
    while (!stack.empty()) {
        const Node *x = stack.back();
        stack.pop_back();
        cached += (int64_t)x->tokens.size();
        if (x->ref == 0) evictable += (int64_t)x->tokens.size();
        stack.insert(stack.end(), x->children.begin(), x->children.end());
    }
    if (out_cached) *out_cached = cached;
    if (out_evictable) *out_evictable = evictable;
    return SGL_OK;
}

int sgl_radix_match_batch(sgl_radix *t, const int32_t *tokens, const int64_t *off, int32_t batch,
                          int32_t lock, int32_t *out_slots, int64_t *out_len, uint64_t *out_node) {
    if (!t || batch < 0 || (batch > 0 && (!off || !out_len))) return SGL_ERR_INVALID;
    for (int32_t r = 0; r < batch; r++)
        if (off[r] < 0 || off[r + 1] < off[r]) return SGL_ERR_INVALID;
    for (int32_t r = 0; r < batch; r++) {
        uint64_t node = 0;
        int rc = sgl_radix_match(t, tokens + off[r], off[r + 1] - off[r], out_slots ? out_slots + off[r] : nullptr,
                                 &out_len[r], &node);
        if (rc != SGL_OK) return rc;
        if (lock && (rc = sgl_radix_lock(t, node, +1)) != SGL_OK) return rc;
        if (out_node) out_node[r] = node;
    }
    return SGL_OK;
}

int sgl_radix_insert_batch(sgl_radix *t, const int32_t *tokens, const int32_t *slots, const int64_t *off,
                           int32_t batch, sgl_kv_pool *pool, int64_t *out_cached_len) {
    if (!t || batch < 0 || (batch > 0 && !off)) return SGL_ERR_INVALID;
    for (int32_t r = 0; r < batch; r++) {
        if (off[r] < 0 || off[r + 1] < off[r]) return SGL_ERR_INVALID;
        int rc = sgl_radix_insert(t, tokens + off[r], slots + off[r], off[r + 1] - off[r], pool,
                                  out_cached_len ? &out_cached_len[r] : nullptr);
        if (rc != SGL_OK) return rc;
    }
    return SGL_OK;
}

int sgl_radix_lock_batch(sgl_radix *t, const uint64_t *nodes, int32_t batch, int32_t delta) {
    if (!t || batch < 0 || (batch > 0 && !nodes) || (delta != 1 && delta != -1)) return SGL_ERR_INVALID;
    return guarded([&] {
        // check everything first (a node may appear several times)
        std::unordered_map<Node *, int64_t> change;
        for (int32_t r = 0; r < batch; r++) {
            if (nodes[r] == 0) continue;
            auto it = t->by_id.find(nodes[r]);
            if (it == t->by_id.end()) return (int)SGL_ERR_INVALID;
            for (Node *x = it->second; x && x != &t->root; x = x->parent) change[x] += delta;
        }
        for (auto &kv : change)
            if (kv.first->ref + kv.second < 0) return (int)SGL_ERR_INVALID;
        for (auto &kv : change) kv.first->ref += kv.second;
        return (int)SGL_OK;
    });
}

int sgl_kv_pool_alloc_batch(sgl_kv_pool *pool, const int64_t *cur_len, const int32_t *last_slot,
                            const int64_t *n, int32_t batch, int32_t *out_slots) {
    if (!pool || batch < 0 || (batch > 0 && (!cur_len || !last_slot || !n))) return SGL_ERR_INVALID;
    const int32_t p = pool->page;
    int64_t need_pages = 0, total = 0;
    // every request's arguments and the page count are checked before any
    // page is popped, so a failing call leaves the pool unchanged
    for (int32_t r = 0; r < batch; r++) {
        if (n[r] < 0 || cur_len[r] < 0) return SGL_ERR_INVALID;
        const int64_t fill = partial_fill(pool, cur_len[r], last_slot[r], n[r]);
        if (fill < 0) return SGL_ERR_INVALID;
        need_pages += (n[r] - fill + p - 1) / p;
        total += n[r];
    }
    if (total > 0 && !out_slots) return SGL_ERR_INVALID;
    if (need_pages > (int64_t)pool->free_pages.size()) return SGL_ERR_OOM;
    int64_t o = 0;
    for (int32_t r = 0; r < batch; r++) {
        const int rc = sgl_kv_pool_alloc(pool, cur_len[r], last_slot[r], n[r], out_slots + o);
        if (rc != SGL_OK) return rc;   // cannot happen: every check above passed
        o += n[r];
    }
    return SGL_OK;
}

}  // extern "C"
