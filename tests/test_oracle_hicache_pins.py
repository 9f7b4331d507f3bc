"""Pins for the host-tier row moves of the oracle (oracle/hicache.py).

The moves are row gathers (HiCache: GPU memory is the first tier, host memory
the second; "SGLang：从前端 DSL 到 SRT 服务运行时", section "从 2024 年论文到今天的
缓存栈").  Each pin below fixes the loop against something other than itself:
slicing for the identity mapping, numpy fancy-index assignment (a library
primitive) for random distinct destinations, the round trip store -> load,
and byte preservation for FP8 codes including NaN patterns.
"""
import numpy as np
import pytest

from oracle import hicache


def _tier(rng, rows, Hkv=2, D=8, dtype=np.float32):
    if dtype == np.uint8:
        return rng.integers(0, 256, (rows, Hkv, D), dtype=np.uint8)
    return rng.standard_normal((rows, Hkv, D)).astype(dtype)


def test_identity_mapping_is_a_slice_copy():
    rng = np.random.default_rng(0)
    pool, host = _tier(rng, 50), _tier(rng, 30)
    n = 17
    out = hicache.load(pool, host, np.arange(n), np.arange(n))
    assert np.array_equal(out[:n], host[:n])
    assert np.array_equal(out[n:], pool[n:])
    back = hicache.store(host, pool, np.arange(n), np.arange(n))
    assert np.array_equal(back[:n], pool[:n])
    assert np.array_equal(back[n:], host[n:])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_gather_matches_fancy_indexing(seed):
    rng = np.random.default_rng(seed)
    pool, host = _tier(rng, 200), _tier(rng, 120)
    n = 64
    slots = rng.permutation(200)[:n]          # distinct destinations
    host_rows = rng.integers(0, 120, n)       # sources may repeat
    ref = pool.copy()
    ref[slots] = host[host_rows]
    assert np.array_equal(hicache.load(pool, host, host_rows, slots), ref)
    hrows = rng.permutation(120)[:n]
    src = rng.integers(0, 200, n)
    ref = host.copy()
    ref[hrows] = pool[src]
    assert np.array_equal(hicache.store(host, pool, src, hrows), ref)


def test_store_then_load_restores_the_rows():
    # evict rows to the host tier, clobber the slots, load them back
    rng = np.random.default_rng(4)
    pool, host = _tier(rng, 100), _tier(rng, 80)
    slots = rng.permutation(100)[:40]
    hrows = rng.permutation(80)[:40]
    host2 = hicache.store(host, pool, slots, hrows)
    clobbered = pool.copy()
    clobbered[slots] = 0
    assert np.array_equal(hicache.load(clobbered, host2, hrows, slots), pool)


def test_fp8_codes_move_unchanged():
    # every byte value, NaN codes 0x7f/0xff included, survives both moves
    rng = np.random.default_rng(5)
    pool = np.zeros((4, 2, 128), np.uint8)
    host = (np.arange(512) % 256).astype(np.uint8).reshape(2, 2, 128)   # all 256 codes, twice
    out = hicache.load(pool, host, np.array([1, 0]), np.array([3, 2]))
    assert np.array_equal(out[3], host[1]) and np.array_equal(out[2], host[0])
    assert np.array_equal(out[:2], pool[:2])
    h2 = hicache.store(_tier(rng, 3, D=128, dtype=np.uint8), out, np.array([2, 3]), np.array([2, 0]))
    assert np.array_equal(h2[2], host[0]) and np.array_equal(h2[0], host[1])


def test_empty_move_is_a_copy():
    rng = np.random.default_rng(6)
    pool, host = _tier(rng, 5), _tier(rng, 5)
    e = np.zeros(0, np.int64)
    out = hicache.load(pool, host, e, e)
    assert np.array_equal(out, pool) and out is not pool
