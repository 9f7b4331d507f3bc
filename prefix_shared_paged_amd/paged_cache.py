"""PagedKVCache: the device pools, the req_to_token table and their host
bookkeeping (slot pool + radix tree), driven through the C ABI.

One request's life, as the pages describe it ("SGLang 深度解读"
(luoboask.github.io) module 2 scheduler and module 5 RadixAttention;
"SGLang 深度拆解" (chenxutan.com) section 2.3):
  admit    -- longest-prefix match in the tree, lock the matched path, write
              the matched slots into the request's req_to_token row;
  append   -- allocate slots for new tokens and append them to the row
              (extend chunks, decode tokens);
  insert   -- put the request's tokens and slots into the tree once its
              prefill completes, so later requests share them;
  release  -- unlock the path and return the request's unshared slots.
All device work (req_to_token scatter, KV store) runs in the library's
kernels; this class only marshals host arrays.
"""
import numpy as np

from . import KVPool, RadixTree, build_req_to_token, store_kv, store_kv_fp8


class Row:
    __slots__ = ("row", "slots", "matched", "node", "tokens", "inserted")

    def __init__(self, row, slots, matched, node, tokens):
        self.row = row
        self.slots = slots        # host int32 slots of positions 0 .. len-1
        self.matched = matched    # cached prefix length at admission
        self.node = node          # locked tree node (0 = none)
        self.tokens = tokens
        self.inserted = 0         # tokens of this row handed to the tree


class PagedKVCache:
    """dtype: the K/V values handed to store(); the pools hold that dtype, or
    e4m3fn codes (uint8) when kv_scale = (k_scale, v_scale) gives the per-KV-head
    factors of an FP8 cache (float32 [Hkv] each)."""

    def __init__(self, num_slots, page_size, Hkv, D, dtype, max_rows, row_stride,
                 init_order=None, device="cuda", kv_scale=None):
        import torch
        self.torch = torch
        self.device = device
        self.Hkv, self.D, self.dtype = Hkv, D, dtype
        self.page_size = page_size
        self.fp8 = kv_scale is not None
        pool_dtype = torch.uint8 if self.fp8 else dtype
        self.k_pool = torch.zeros((num_slots, Hkv, D), dtype=pool_dtype, device=device)
        self.v_pool = torch.zeros((num_slots, Hkv, D), dtype=pool_dtype, device=device)
        if self.fp8:
            self.k_scale = self._dev(np.asarray(kv_scale[0], np.float32).reshape(Hkv), torch.float32)
            self.v_scale = self._dev(np.asarray(kv_scale[1], np.float32).reshape(Hkv), torch.float32)
        self.r2t = torch.full((max_rows, row_stride), -1, dtype=torch.int32, device=device)
        self.pool = KVPool(num_slots, page_size, init_order)
        self.tree = RadixTree(page_size)
        self.free_rows = list(range(max_rows))
        self.rows = {}

    # -- helpers -------------------------------------------------------------
    def _dev(self, a, dtype):
        return self.torch.as_tensor(np.ascontiguousarray(a), dtype=dtype).to(self.device, non_blocking=False)

    @staticmethod
    def _csr(parts):
        off = np.zeros(len(parts) + 1, np.int64)
        off[1:] = np.cumsum([len(p) for p in parts])
        flat = np.concatenate(parts).astype(np.int32) if parts and off[-1] > 0 else np.zeros(1, np.int32)
        return flat, off

    # -- request life --------------------------------------------------------
    def admit(self, token_lists, lock=True):
        """Match each token list, lock its path, write the matched slots to a fresh row."""
        rows, prefixes = [], []
        for toks in token_lists:
            n, slots, node = self.tree.match(toks)
            if lock and node:
                self.tree.lock(node, +1)
            r = self.free_rows.pop(0)
            st = Row(r, slots.astype(np.int32), n, node if lock else 0, np.asarray(toks, np.int32))
            self.rows[r] = st
            rows.append(st)
            prefixes.append(st.slots)
        flat, off = self._csr(prefixes)
        empty = np.zeros(1, np.int32)
        build_req_to_token(self.r2t, self._dev([s.row for s in rows], self.torch.int32),
                           self._dev(empty, self.torch.int32),
                           self._dev(np.zeros(len(rows) + 1, np.int64), self.torch.int64),
                           prefix_slots=self._dev(flat, self.torch.int32),
                           prefix_off=self._dev(off, self.torch.int64))
        return rows

    def append(self, rows, counts):
        """Allocate counts[i] slots for rows[i] and append them to its req_to_token row."""
        news, col0 = [], []
        for st, n in zip(rows, counts):
            cur = len(st.slots)
            last = int(st.slots[-1]) if cur else -1
            new = self.pool.alloc(int(n), cur, last)
            col0.append(cur)
            st.slots = np.concatenate([st.slots, new]).astype(np.int32)
            news.append(new)
        flat, off = self._csr(news)
        build_req_to_token(self.r2t, self._dev([s.row for s in rows], self.torch.int32),
                           self._dev(flat, self.torch.int32), self._dev(off, self.torch.int64),
                           new_col0=self._dev(col0, self.torch.int32))
        return news

    def store(self, k, v, slots):
        """Store K/V rows (device tensors [n, Hkv, D]) at host slot ids."""
        if len(slots) == 0:
            return
        if self.fp8:
            store_kv_fp8(k, v, self._dev(slots, self.torch.int32), self.k_pool, self.v_pool, self.k_scale,
                         self.v_scale)
        else:
            store_kv(k, v, self._dev(slots, self.torch.int32), self.k_pool, self.v_pool)

    def insert(self, st, n_tokens=None):
        """Insert the row's first n_tokens (whole pages) into the tree once its
        prefill completes, and move the row's lock to the new end of its path.
        Returns how many of those tokens the tree already held."""
        n = len(st.tokens) if n_tokens is None else n_tokens
        n = min(n, len(st.slots))
        cached = self.tree.insert(st.tokens[:n], st.slots[:n], self.pool)
        n_ins = n // self.page_size * self.page_size
        st.inserted = max(st.inserted, n_ins)
        if st.node or n_ins:
            m, slots, node = self.tree.match(st.tokens[:n_ins])
            # The tree's slots win for pages it held before (the row's duplicates
            # were freed): point the row's req_to_token entries at them.
            if not np.array_equal(slots, st.slots[:m]):
                build_req_to_token(self.r2t, self._dev([st.row], self.torch.int32),
                                   self._dev(slots, self.torch.int32),
                                   self._dev([0, m], self.torch.int64),
                                   new_col0=self._dev([0], self.torch.int32))
            st.slots = np.concatenate([slots, st.slots[m:]]).astype(np.int32)
            if node:
                self.tree.lock(node, +1)
            if st.node:
                self.tree.lock(st.node, -1)
            st.node = node
        return cached

    def release(self, st):
        """Unlock the row's path and free the slots the tree does not hold."""
        if st.node:
            self.tree.lock(st.node, -1)
        keep = max(st.matched, st.inserted)
        mine = st.slots[keep:]
        if len(mine):
            self.pool.free(mine)
        del self.rows[st.row]
        self.free_rows.append(st.row)

    # -- device views ----------------------------------------------------------
    def rows_tensor(self, rows):
        return self._dev([s.row for s in rows], self.torch.int32)
