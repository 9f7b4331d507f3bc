"""Brute-force model of the prefix cache (radix tree) and the KV slot pool.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Deliberately the most
direct data structure: an UNCOMPRESSED trie with one page of tokens per edge
(one token per edge at page size 1), the shape of the match / insert pseudo
code in "SGLang 深度拆解" (chenxutan.com) section 2.3 and of the TreeNode
pseudo source in "SGLang 深度解读" (luoboask.github.io), module 1 RadixCache.
The product's tree is a compressed radix tree (multi-token edges, the form
described in bhfrc.com news 45689 section 3.1 and in "SGLang：从前端 DSL 到
SRT 服务运行时" (oripoin.cn), section "用基数树实现前缀复用"); both must give
identical observable results.

Rules (the pages leave the details open; these are the readings used):
  * pages: page size p >= 1; a page is p consecutive slots page*p .. page*p+p-1.
    Sharing happens in whole pages: a match is a whole number of pages.
  * pool: a FIFO free list of page ids, initialised from a caller-given
    order (a seeded permutation).  alloc pops from the head, free appends
    to the tail.  For p > 1, alloc first fills the rest of the request's
    last page, and free takes a slot list and returns the page of every
    slot that starts a page.  A request that needs more pages than are free
    gets an out-of-memory error and the pool is unchanged.
  * clock: a logical clock ticks once per match and once per insert; every
    node on the matched / inserted path is stamped with it.
  * match returns the longest cached prefix (whole pages) and its slots.
  * insert adds the pages not yet cached.  For a page that is already
    cached, the tree keeps its own slots; if the caller's slots for it
    differ, the caller's page is a duplicate and is freed to the pool (in
    position order).  It returns how many tokens were already cached.
  * lock(node, +-1) changes the reference count of every node on the path
    root..node; counts never go below 0.
  * evict(n): repeatedly remove the unreferenced leaf with the oldest stamp,
    freeing its page, until at least n tokens are freed or nothing is
    evictable (leaf-first LRU guarded by reference counts, oripoin.cn section
    "用基数树实现前缀复用" first two bullets; chenxutan.com section 2.3
    _evict).  A parent becomes a leaf when its last child goes.  Two leaves
    never share a stamp (one operation stamps one root path, which holds at
    most one leaf), so the order is unique.
"""
from collections import deque


class OutOfSlots(Exception):
    pass


class SlotPool:
    def __init__(self, num_slots, page_size=1, init_order=None):
        assert num_slots % page_size == 0
        self.p = page_size
        n_pages = num_slots // page_size
        if init_order is None:
            init_order = list(range(n_pages))
        init_order = [int(x) for x in init_order]
        assert sorted(init_order) == list(range(n_pages)), "init_order must be a permutation"
        self.free_pages = deque(init_order)  # head = left end
        self.is_free = [True] * n_pages
        self.num_slots = num_slots

    def available(self):
        return len(self.free_pages) * self.p

    def alloc(self, cur_len, last_slot, n):
        p = self.p
        out = []
        if p > 1 and cur_len % p != 0:
            k = min(n, p - cur_len % p)
            out.extend(last_slot + 1 + i for i in range(k))
        rest = n - len(out)
        need = -(-rest // p)
        if need > len(self.free_pages):
            raise OutOfSlots(f"need {need} pages, {len(self.free_pages)} free")
        for _ in range(need):
            page = self.free_pages.popleft()
            self.is_free[page] = False
            for i in range(p):
                if len(out) < n:
                    out.append(page * p + i)
        return out

    def free(self, slots):
        for s in slots:
            s = int(s)
            if s % self.p != 0:
                continue
            page = s // self.p
            assert not self.is_free[page], f"double free of page {page}"
            self.is_free[page] = True
            self.free_pages.append(page)


class Node:
    __slots__ = ("children", "parent", "page", "slots", "ref", "stamp")

    def __init__(self, parent, page, slots, stamp):
        self.children = {}
        self.parent = parent
        self.page = page          # tuple of p token ids on the edge into this node
        self.slots = slots        # list of p slot ids
        self.ref = 0
        self.stamp = stamp


class PrefixCache:
    def __init__(self, page_size=1):
        self.p = page_size
        self.root = Node(None, None, None, 0)
        self.clock = 0

    def _pages(self, tokens):
        p = self.p
        n = len(tokens) // p * p
        return [tuple(int(t) for t in tokens[i:i + p]) for i in range(0, n, p)]

    def match(self, tokens):
        """Return (matched_len, slots, node)."""
        self.clock += 1
        node = self.root
        slots = []
        for pg in self._pages(tokens):
            child = node.children.get(pg)
            if child is None:
                break
            node = child
            node.stamp = self.clock
            slots.extend(node.slots)
        return len(slots), slots, node

    def insert(self, tokens, slots, pool):
        """Insert whole pages of tokens with their slots; return cached prefix length."""
        self.clock += 1
        p = self.p
        node = self.root
        already = 0
        fresh = False
        for i, pg in enumerate(self._pages(tokens)):
            my_slots = [int(s) for s in slots[i * p:(i + 1) * p]]
            child = None if fresh else node.children.get(pg)
            if child is not None:
                child.stamp = self.clock
                if child.slots[0] != my_slots[0]:
                    pool.free([my_slots[0]])          # the caller's duplicate page
                already += p
                node = child
            else:
                fresh = True
                child = Node(node, pg, my_slots, self.clock)
                node.children[pg] = child
                node = child
        return already

    def lock(self, node, delta):
        path = []
        x = node
        while x is not self.root:
            path.append(x)
            x = x.parent
        if any(n.ref + delta < 0 for n in path):
            raise ValueError("reference count would go negative")
        for n in path:
            n.ref += delta

    def _all_nodes(self):
        stack = list(self.root.children.values())
        while stack:
            n = stack.pop()
            yield n
            stack.extend(n.children.values())

    def evict(self, n_tokens, pool):
        freed = 0
        while freed < n_tokens:
            leaves = [n for n in self._all_nodes() if not n.children and n.ref == 0]
            if not leaves:
                break
            victim = min(leaves, key=lambda n: n.stamp)
            del victim.parent.children[victim.page]
            pool.free([victim.slots[0]])
            freed += self.p
        return freed

    def cached_tokens(self):
        return sum(self.p for _ in self._all_nodes())

    def evictable_tokens(self):
        return sum(self.p for n in self._all_nodes() if n.ref == 0)


def expected_req_to_token(rows, num_rows, row_stride, fill=-1):
    """Plain expected req_to_token table: rows = {row_index: slot list}."""
    import numpy as np
    t = np.full((num_rows, row_stride), fill, np.int32)
    for r, slots in rows.items():
        t[r, :len(slots)] = slots
    return t
