"""Pins of the brute-force prefix-cache / slot-pool model (oracle/radix_model.py).

- worked examples printed on the pages (tests/golden/radix_worked_examples.json);
- the plain definition of a match: the longest common prefix with any cached
  sequence, in whole pages, checked on random small-alphabet sequences;
- hand cases of the allocator (FIFO order, partial pages, out-of-memory).
"""
import json
import os

import numpy as np
import pytest

from oracle.radix_model import OutOfSlots, PrefixCache, SlotPool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "radix_worked_examples.json")) as f:
        return json.load(f)


def _insert_request(tree, pool, toks):
    n, slots, node = tree.match(toks)
    new = pool.alloc(n, slots[-1] if slots else -1, len(toks) - n)
    tree.insert(toks, list(slots) + list(new), pool)
    return n


def test_shared_system_prompt_example():
    g = _golden()["shared_system_prompt"]
    pool = SlotPool(1024)
    tree = PrefixCache()
    sys_t = list(range(1, g["system_tokens"] + 1))
    for i, u in enumerate(g["unique_tokens"]):
        toks = sys_t + [1000 + 100 * i + j for j in range(u)]
        _insert_request(tree, pool, toks)
    assert tree.cached_tokens() == g["expected_cached_tokens"]
    per_request = sum(g["system_tokens"] + u for u in g["unique_tokens"])
    assert per_request - tree.cached_tokens() == g["expected_saved_tokens"]
    n, slots, _ = tree.match(sys_t + [9999])
    assert n == g["fourth_request_match"]
    assert 1024 - pool.available() == tree.cached_tokens()


def test_ten_requests_one_prompt():
    g = _golden()["ten_requests_one_prompt"]
    pool = SlotPool(8192)
    tree = PrefixCache()
    sys_t = list(range(1, g["system_tokens"] + 1))
    got = []
    for i in range(g["n_requests"]):
        toks = sys_t + [50000 + 100 * i + j for j in range(g["user_tokens"])]
        got.append(_insert_request(tree, pool, toks))
    assert got == g["expected_match_lengths"]


def test_figure_tree_shape_and_leaves():
    g = _golden()["figure_tree"]
    seg = {}
    nxt = 1
    for name, n in g["segments"].items():
        seg[name] = list(range(nxt, nxt + n))
        nxt += n
    pool = SlotPool(256)
    tree = PrefixCache()
    for path in g["paths"]:
        toks = [t for s in path for t in seg[s]]
        _insert_request(tree, pool, toks)
    assert tree.cached_tokens() == sum(g["segments"].values())
    # the leaves are the last tokens of the three leaf segments
    leaves = sorted(n.page[0] for n in tree._all_nodes() if not n.children)
    assert leaves == sorted(seg[s][-1] for s in g["leaves"])
    # partial matches stop at the divergence point
    n, _, _ = tree.match(seg["System"] + seg["Q1+R1"] + seg["Q2+R2"])
    assert n == len(seg["System"]) + len(seg["Q1+R1"])
    n, _, _ = tree.match(seg["System"][:3] + [9999])
    assert n == 3


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


@pytest.mark.parametrize("p", [1, 2, 4])
def test_match_is_longest_common_prefix_in_whole_pages(p):
    rng = np.random.default_rng(123 + p)
    pool = SlotPool(4096, p)
    tree = PrefixCache(p)
    inserted = []
    inserted_slots = []
    for it in range(300):
        toks = list(rng.integers(0, 3, size=rng.integers(0, 14)))
        n, slots, _ = tree.match(toks)
        want = max([_lcp(toks, s) // p * p for s in inserted] + [0])
        assert n == want
        # the returned slots are the slots the cache holds for that prefix
        for s, sl in inserted_slots:
            m = _lcp(toks, s) // p * p
            if m == n and n > 0:
                assert slots == sl[:n]
                break
        if rng.random() < 0.5:
            new = pool.alloc(n, slots[-1] if slots else -1, len(toks) - n)
            full = slots + new
            tree.insert(toks, full, pool)
            ins = len(toks) // p * p
            if ins:
                inserted.append(toks[:ins])
                inserted_slots.append((toks[:ins], full[:ins]))
            # free the request's unshared tail (partial page)
            pool.free(full[ins:])


def test_allocator_fifo_and_pages():
    pool = SlotPool(16, 4, init_order=[2, 0, 3, 1])
    a = pool.alloc(0, -1, 6)                 # page 2 -> 8..11, page 0 -> 0,1
    assert a == [8, 9, 10, 11, 0, 1]
    b = pool.alloc(6, 1, 3)                  # fill page 0 (2, 3), then page 3 -> 12
    assert b == [2, 3, 12]
    assert pool.available() == 4
    with pytest.raises(OutOfSlots):
        pool.alloc(0, -1, 5)
    assert pool.available() == 4             # unchanged by the failed request
    pool.free(a + b)                         # pages 2, 0, 3 back in slot order
    assert list(pool.free_pages) == [1, 2, 0, 3]
    c = pool.alloc(0, -1, 1)
    assert c == [4]


def test_eviction_is_leaf_first_lru_and_respects_refs():
    pool = SlotPool(64)
    tree = PrefixCache()
    A = [1, 2, 3, 4]
    Bq = [1, 2, 7, 8, 9]
    C = [5, 6]
    for t in (A, Bq, C):
        _insert_request(tree, pool, t)
    assert tree.cached_tokens() == 4 + 3 + 2
    n, _, node_b = tree.match(Bq)            # B is now the most recent
    tree.lock(node_b, +1)
    freed = tree.evict(3, pool)              # oldest leaf is A's tail (3, 4), then C
    assert freed == 3
    assert tree.match(A)[0] == 2             # A's own tail is gone, shared [1, 2] stays
    assert tree.match(C)[0] == 1
    freed = tree.evict(100, pool)            # everything unreferenced
    assert tree.match(Bq)[0] == 5            # locked path survives
    assert tree.cached_tokens() == 5
    tree.lock(node_b, -1)
    assert tree.evict(100, pool) == 5
    assert tree.cached_tokens() == 0
    assert pool.available() == 64
    with pytest.raises(ValueError):
        tree.lock(node_b, -1)


def test_duplicate_pages_are_freed_on_insert():
    pool = SlotPool(32)
    tree = PrefixCache()
    toks = [3, 1, 4, 1, 5]
    s1 = pool.alloc(0, -1, 5)
    s2 = pool.alloc(0, -1, 5)                # a second request computed the same tokens
    assert tree.insert(toks, s1, pool) == 0
    before = pool.available()
    assert tree.insert(toks, s2, pool) == 5  # all already cached
    assert pool.available() == before + 5    # the second copy went back to the pool
    assert list(pool.free_pages)[-5:] == s2
    assert tree.match(toks)[1] == s1
