"""Host bookkeeping of the library (compressed radix tree + slot pool, C++)
against the brute-force model in oracle/radix_model.py (an uncompressed trie),
bit-exact: match lengths and slots, cached-prefix lengths on insert, freed
counts on evict, tree statistics and the pool's free-list order.
"""
import numpy as np
import pytest

import prefix_shared_paged_amd as sp
from oracle.radix_model import OutOfSlots, PrefixCache, SlotPool


def _drain(pool_lib, pool_model):
    """Compare the two free lists by allocating everything that is left."""
    n = pool_model.available()
    assert pool_lib.available() == n
    if n == 0:
        return
    got = pool_lib.alloc(n)
    want = pool_model.alloc(0, -1, n)
    np.testing.assert_array_equal(got, np.asarray(want, np.int32))


@pytest.mark.parametrize("p,seed", [(1, 0), (1, 1), (2, 2), (4, 3), (16, 4)])
def test_random_operations_match_model(p, seed):
    rng = np.random.default_rng(seed)
    n_slots = 4096 if p < 16 else 16384
    order = rng.permutation(n_slots // p).astype(np.int32)
    pool_l, pool_m = sp.KVPool(n_slots, p, order), SlotPool(n_slots, p, order)
    tree_l, tree_m = sp.RadixTree(p), PrefixCache(p)
    vocab = 3 if p == 1 else 2
    live = []            # (lib handle, model node, tokens, slots, matched)
    for step in range(2500):
        op = rng.random()
        if op < 0.45:
            # a request: match, maybe lock, allocate, maybe insert, maybe release now
            L = int(rng.integers(0, 6 * p + 3))
            toks = rng.integers(0, vocab, size=L).astype(np.int32)
            n_l, s_l, node_l = tree_l.match(toks)
            n_m, s_m, node_m = tree_m.match(toks)
            assert n_l == n_m
            np.testing.assert_array_equal(s_l, np.asarray(s_m, np.int32))
            cur_last = int(s_l[-1]) if n_l else -1
            try:
                new_m = pool_m.alloc(n_m, cur_last, L - n_m)
                oom = False
            except OutOfSlots:
                oom = True
            if oom:
                with pytest.raises(sp.OutOfSlots):
                    pool_l.alloc(L - n_l, n_l, cur_last)
                continue
            new_l = pool_l.alloc(L - n_l, n_l, cur_last)
            np.testing.assert_array_equal(new_l, np.asarray(new_m, np.int32))
            slots = np.concatenate([s_l, new_l]).astype(np.int32)
            if rng.random() < 0.7:
                c_l = tree_l.insert(toks, slots, pool_l)
                c_m = tree_m.insert(toks, slots, pool_m)
                assert c_l == c_m
                ins = L // p * p
                # the unshared tail (partial page) goes back to the pool now
                pool_l.free(slots[ins:])
                pool_m.free(slots[ins:])
            else:
                pool_l.free(slots[n_l:])
                pool_m.free(slots[n_m:])
            if rng.random() < 0.3 and n_l > 0:
                tree_l.lock(node_l, +1)
                tree_m.lock(node_m, +1)
                live.append((node_l, node_m))
        elif op < 0.55 and live:
            i = int(rng.integers(0, len(live)))
            node_l, node_m = live.pop(i)
            tree_l.lock(node_l, -1)
            tree_m.lock(node_m, -1)
        elif op < 0.75:
            want = int(rng.integers(0, 8 * p))
            f_l = tree_l.evict(want, pool_l)
            f_m = tree_m.evict(want, pool_m)
            assert f_l == f_m
        else:
            # a request with a duplicate computation of an already cached sequence
            L = int(rng.integers(1, 4 * p + 1))
            toks = rng.integers(0, vocab, size=L).astype(np.int32)
            try:
                slots_m = pool_m.alloc(0, -1, L)
            except OutOfSlots:
                with pytest.raises(sp.OutOfSlots):
                    pool_l.alloc(L)
                continue
            slots_l = pool_l.alloc(L)
            np.testing.assert_array_equal(slots_l, np.asarray(slots_m, np.int32))
            assert tree_l.insert(toks, slots_l, pool_l) == tree_m.insert(toks, slots_l, pool_m)
            ins = L // p * p
            pool_l.free(slots_l[ins:])
            pool_m.free(slots_l[ins:])
        if step % 50 == 0:
            assert tree_l.stats() == (tree_m.cached_tokens(), tree_m.evictable_tokens())
            assert pool_l.available() == pool_m.available()
    for node_l, node_m in live:
        tree_l.lock(node_l, -1)
        tree_m.lock(node_m, -1)
    assert tree_l.evict(10 ** 9, pool_l) == tree_m.evict(10 ** 9, pool_m)
    assert tree_l.stats() == (0, 0)
    _drain(pool_l, pool_m)


def test_pool_errors_leave_pool_unchanged():
    pool = sp.KVPool(8, 2, [3, 1, 0, 2])
    a = pool.alloc(3)                       # pages 3, 1 -> 6, 7, 2
    np.testing.assert_array_equal(a, [6, 7, 2])
    with pytest.raises(sp.OutOfSlots):
        pool.alloc(5)
    assert pool.available() == 4
    with pytest.raises(sp.SglError):
        pool.free([6, 6])                   # same page twice
    with pytest.raises(sp.SglError):
        pool.free([0])                      # page 0 is free already
    with pytest.raises(sp.SglError):
        pool.free([99])                     # out of range
    assert pool.available() == 4
    pool.free(a)
    assert pool.available() == 8
    with pytest.raises(sp.SglError):
        sp.KVPool(8, 2, [0, 0, 1, 2])       # not a permutation
    with pytest.raises(sp.SglError):
        sp.KVPool(9, 2)                     # not a whole number of pages


def test_tree_errors_leave_tree_unchanged():
    pool = sp.KVPool(64, 4)
    tree = sp.RadixTree(4)
    s = pool.alloc(8)
    tree.insert([1, 2, 3, 4, 5, 6, 7, 8], s, pool)
    with pytest.raises(sp.SglError):
        tree.insert([9, 9, 9, 9], [1, 2, 3, 4], pool)      # page not aligned
    with pytest.raises(sp.SglError):
        tree.lock(12345, 1)                                 # unknown node
    n, _, node = tree.match([1, 2, 3, 4, 5, 6, 7, 8])
    with pytest.raises(sp.SglError):
        tree.lock(node, -1)                                 # would go negative
    assert tree.stats() == (8, 8)
    assert n == 8


def test_figure_example_through_library():
    # 'SGLang 深度拆解' section 2.3 figure: after the three requests the tree holds
    # System, Q1+R1, Q2+R2, Q3+R3, Q3b+R3b, Q4+R4 once each.
    seg = {"S": [1, 2, 3], "Q1": [4, 5], "Q2": [6], "Q3": [7, 8], "Q3b": [9], "Q4": [10, 11]}
    pool = sp.KVPool(64)
    tree = sp.RadixTree(1)
    for path in (["S", "Q1", "Q3", "Q4"], ["S", "Q1", "Q3b"], ["S", "Q2"]):
        toks = [t for x in path for t in seg[x]]
        n, slots, _ = tree.match(toks)
        new = pool.alloc(len(toks) - n)
        tree.insert(toks, np.concatenate([slots, new]), pool)
    assert tree.stats() == (sum(len(v) for v in seg.values()),) * 2
    assert tree.match(seg["S"] + seg["Q1"] + seg["Q2"])[0] == 5


def test_batched_calls_equal_sequential_calls():
    rng = np.random.default_rng(11)
    for p in (1, 4):
        order = rng.permutation(2048 // p).astype(np.int32)
        pa, pb = sp.KVPool(2048, p, order), sp.KVPool(2048, p, order)
        ta, tb = sp.RadixTree(p), sp.RadixTree(p)
        for it in range(30):
            B = int(rng.integers(1, 6))
            toks = [rng.integers(0, 3, size=int(rng.integers(0, 5 * p + 2))).astype(np.int32) for _ in range(B)]
            off = np.zeros(B + 1, np.int64)
            off[1:] = np.cumsum([len(t) for t in toks])
            flat = np.concatenate(toks) if off[-1] else np.zeros(0, np.int32)
            sl, lens, nodes = ta.match_batch(flat, off, lock=True)
            singles = []
            for r, t in enumerate(toks):
                n, s1, node = tb.match(t)
                tb.lock(node, +1)
                singles.append((n, s1, node))
                assert lens[r] == n
                np.testing.assert_array_equal(sl[off[r]:off[r] + n], s1)
            need = np.array([len(t) - n for t, (n, _, _) in zip(toks, singles)], np.int64)
            cur = np.array([n for n, _, _ in singles], np.int64)
            last = np.array([int(s1[-1]) if n else -1 for n, s1, _ in singles], np.int32)
            new_a, noff = pa.alloc_batch(need, cur, last)
            new_b = [pb.alloc(int(k), int(c), int(l)) for k, c, l in zip(need, cur, last)]
            np.testing.assert_array_equal(new_a, np.concatenate(new_b) if new_b else new_a)
            full = [np.concatenate([s1, new_a[noff[r]:noff[r + 1]]]) for r, (n, s1, _) in enumerate(singles)]
            ca = ta.insert_batch(flat, np.concatenate(full) if off[-1] else np.zeros(0, np.int32), off, pa)
            cb = [tb.insert(t, f, pb) for t, f in zip(toks, full)]
            np.testing.assert_array_equal(ca, cb)
            for r, t in enumerate(toks):
                ins = len(t) // p * p
                pa.free(full[r][ins:])
                pb.free(full[r][ins:])
            ta.lock_batch(nodes, -1)
            for _, _, node in singles:
                tb.lock(node, -1)
            assert ta.stats() == tb.stats()
            assert pa.available() == pb.available()
            want = int(rng.integers(0, 6))
            assert ta.evict(want, pa) == tb.evict(want, pb)


def test_batched_alloc_is_all_or_nothing():
    pool = sp.KVPool(64, 4)
    with pytest.raises(sp.OutOfSlots):
        pool.alloc_batch([32, 40], [0, 0], [-1, -1])
    assert pool.available() == 64
    a, off = pool.alloc_batch([3, 5], [0, 0], [-1, -1])
    assert off.tolist() == [0, 3, 8] and pool.available() == 64 - 12


def test_batched_alloc_rejects_a_bad_request_before_popping():
    # request 1's last slot cannot end a 3-token request on 4-slot pages: the
    # batch fails as a whole, request 0's pages stay in the pool, and the free
    # list keeps its order (the next allocation gets the same slots)
    pool = sp.KVPool(64, 4)
    first, _ = pool.alloc_batch([4], [0], [-1])
    pool.free(first)
    with pytest.raises(sp.SglError) as e:
        pool.alloc_batch([5, 2], [0, 3], [-1, 9])
    assert e.value.status == sp.SGL_ERR_INVALID
    assert pool.available() == 64
    again, _ = pool.alloc_batch([5], [0], [-1])
    ref = sp.KVPool(64, 4)
    ref.alloc_batch([4], [0], [-1])
    ref.free(first)
    want, _ = ref.alloc_batch([5], [0], [-1])
    np.testing.assert_array_equal(again, want)
