"""GPU parity of the host-tier row moves (HiCache prefetch / write-back), through the C ABI.

Host tiers are page-locked CPU tensors; pools are device tensors.  Row
contents are random bit patterns (every bf16 / fp8 code may appear, NaN codes
included), so the check is bit for bit against oracle/hicache.py on the same
seeded arrays: the moved rows and every row that must stay untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

import prefix_shared_paged_amd as sp
from oracle import hicache

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _bits(shape, dtype, rng):
    """Random contents as raw bits: int16 for bf16, uint8 for fp8 codes, int32 for f32."""
    if dtype == torch.bfloat16:
        return torch.from_numpy(rng.integers(-32768, 32768, shape, dtype=np.int16)).view(torch.bfloat16)
    if dtype == torch.uint8:
        return torch.from_numpy(rng.integers(0, 256, shape, dtype=np.uint8))
    return torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31, shape, dtype=np.int32)).view(torch.float32)


def _np(t):
    """Raw bits of a tensor as a numpy array (device tensors are copied back)."""
    t = t.cpu() if t.is_cuda else t
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().copy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().copy()
    return t.numpy().copy()


def _tiers(seed, row_shape, dtype, num_slots, n_host, two):
    rng = np.random.default_rng(seed)
    pools = [_bits((num_slots,) + row_shape, dtype, rng).cuda() for _ in range(1 + two)]
    hosts = []
    for _ in range(1 + two):
        h = torch.empty((n_host,) + row_shape, dtype=dtype, pin_memory=True)
        h.copy_(_bits((n_host,) + row_shape, dtype, rng))
        hosts.append(h)
    return rng, pools, hosts


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


CASES = [
    # (row shape, dtype, K and V?) -- bf16 Hkv 8 D 128 (2 KiB rows), FP8 codes,
    # fp32 Hkv 2 D 64 (512 B), one latent tier of 576 bf16 (1152 B: 72 chunks)
    ((8, 128), torch.bfloat16, True),
    ((8, 128), torch.uint8, True),
    ((2, 64), torch.float32, True),
    ((576,), torch.bfloat16, False),
]


@pytest.mark.parametrize("row_shape,dtype,two", CASES)
@pytest.mark.parametrize("n", [1, 777])
def test_prefetch_and_write_back_match_the_oracle(row_shape, dtype, two, n):
    num_slots, n_host = 4096, 1500
    rng, pools, hosts = _tiers(n + len(row_shape), row_shape, dtype, num_slots, n_host, two)
    _print(f"hicache rows {row_shape} {dtype} two={two} n={n}")
    # prefetch: distinct destination slots, host rows may repeat
    slots = rng.permutation(num_slots)[:n]
    hrows = rng.integers(0, n_host, n)
    before = [_np(p) for p in pools]
    sp.hicache_prefetch(hosts[0], hosts[1] if two else None, _dev(hrows, torch.int64), _dev(slots, torch.int32),
                        pools[0], pools[1] if two else None)
    torch.cuda.synchronize()
    for p, h, b in zip(pools, hosts, before):
        assert np.array_equal(_np(p), hicache.load(b, _np(h), hrows, slots))
    # write-back: distinct destination host rows, slots may repeat
    hrows = rng.permutation(n_host)[:n]
    slots = rng.integers(0, num_slots, n)
    before = [_np(h) for h in hosts]
    sp.hicache_write_back(pools[0], pools[1] if two else None, _dev(slots, torch.int32), _dev(hrows, torch.int64),
                          hosts[0], hosts[1] if two else None)
    torch.cuda.synchronize()
    for p, h, b in zip(pools, hosts, before):
        assert np.array_equal(_np(h), hicache.store(b, _np(p), slots, hrows))


def test_round_trip_through_the_host_tier():
    # evict rows to the host tier, clobber their slots, prefetch them back
    num_slots, n_host, n = 8192, 3000, 2500
    rng, pools, hosts = _tiers(7, (8, 128), torch.bfloat16, num_slots, n_host, True)
    slots = _dev(rng.permutation(num_slots)[:n], torch.int32)
    hrows = _dev(rng.permutation(n_host)[:n], torch.int64)
    keep = [p.clone() for p in pools]
    sp.hicache_write_back(pools[0], pools[1], slots, hrows, hosts[0], hosts[1])
    for p in pools:
        p[slots.long()] = 0
    sp.hicache_prefetch(hosts[0], hosts[1], hrows, slots, pools[0], pools[1])
    torch.cuda.synchronize()
    for p, k in zip(pools, keep):
        assert torch.equal(p.view(torch.int16), k.view(torch.int16))


def test_out_of_range_moves_are_skipped():
    # indices outside a buffer are skipped by the kernel's own bounds checks
    num_slots, n_host = 512, 300
    rng, pools, hosts = _tiers(11, (8, 128), torch.bfloat16, num_slots, n_host, True)
    slots = np.array([3, num_slots, 7, 9, -5], np.int64)
    hrows = np.array([10, 11, -1, n_host, 12], np.int64)
    before = [_np(p) for p in pools]
    sp.hicache_prefetch(hosts[0], hosts[1], _dev(hrows, torch.int64), _dev(slots, torch.int32), pools[0], pools[1])
    torch.cuda.synchronize()
    for p, h, b in zip(pools, hosts, before):
        assert np.array_equal(_np(p), hicache.load(b, _np(h), hrows[:1], slots[:1]))
    hb = [_np(h) for h in hosts]
    sp.hicache_write_back(pools[0], pools[1], _dev(slots, torch.int32), _dev(hrows, torch.int64), hosts[0], hosts[1])
    torch.cuda.synchronize()
    for p, h, b in zip(pools, hosts, hb):
        assert np.array_equal(_np(h), hicache.store(b, _np(p), slots[:1], hrows[:1]))


def test_unpinned_or_device_host_tier_is_rejected():
    lib = sp.load()
    pool = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device="cuda")
    idx_i = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx_l = torch.zeros(4, dtype=torch.int64, device="cuda")
    pageable = torch.zeros((64, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sp.hicache_prefetch(pageable, None, idx_l, idx_i, pool)
    # the library's own check, past the binding: pageable memory, device memory,
    # and a pinned buffer shorter than the stated tier
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for host, rows in ((pageable, 64), (pool, 64)):
        assert lib.sgl_hicache_prefetch(P(host), None, rows, P(idx_l), P(idx_i), 4, P(pool), None, 64, 2048,
                                        None) == sp.SGL_ERR_INVALID
    small = torch.zeros((16, 8, 128), dtype=torch.bfloat16, pin_memory=True)
    big_rows = 1 << 30  # far past the end of the pinned allocation
    assert lib.sgl_hicache_write_back(P(pool), None, 64, P(idx_i), P(idx_l), 4, P(small), None, big_rows, 2048,
                                      None) == sp.SGL_ERR_INVALID
    assert lib.sgl_hicache_prefetch(P(small), None, 16, P(idx_l), P(idx_i), 0, P(pool), None, 64, 2048,
                                    None) == sp.SGL_OK
    torch.cuda.synchronize()
    assert int(pool.view(torch.int16).abs().sum()) == 0


def test_prefetch_at_full_size():
    # the throughput workload's shape: 65,536 scattered rows of one layer's
    # K and V (8 KV heads x 128 bf16) from a 2^18-row host tier into a
    # 2^20-slot pool
    num_slots, n_host, n = 1 << 20, 1 << 18, 65536
    rng = np.random.default_rng(5)
    _print("hicache full size: building tiers")
    pools = [torch.empty((num_slots, 8, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for p in pools:
        p.view(torch.int16).random_(-32768, 32767)
    hosts = []
    for _ in range(2):
        h = torch.empty((n_host, 8, 128), dtype=torch.bfloat16, pin_memory=True)
        h.view(torch.int16).copy_(torch.from_numpy(rng.integers(-32768, 32768, (n_host, 8, 128), dtype=np.int16)))
        hosts.append(h)
    slots = rng.permutation(num_slots)[:n]
    hrows = rng.permutation(n_host)[:n]
    sl_d, hr_d = _dev(slots, torch.int32), _dev(hrows, torch.int64)
    untouched = _dev(np.setdiff1d(rng.integers(0, num_slots, 4096), slots), torch.int64)
    before = [_np(p[untouched]) for p in pools]
    sp.hicache_prefetch(hosts[0], hosts[1], hr_d, sl_d, pools[0], pools[1])
    torch.cuda.synchronize()
    # every moved row, bit for bit, plus a sample of untouched slots
    for p, h in zip(pools, hosts):
        got = _np(p[sl_d.long()])
        assert np.array_equal(got, hicache.load(np.zeros_like(got), _np(h), hrows, np.arange(n)))
    # write the same rows back to fresh host rows and compare
    hrows2 = (hrows + 7) % n_host
    hb = [_np(h) for h in hosts]
    sp.hicache_write_back(pools[0], pools[1], sl_d, _dev(hrows2, torch.int64), hosts[0], hosts[1])
    torch.cuda.synchronize()
    for p, h, b in zip(pools, hosts, hb):
        assert np.array_equal(_np(h), hicache.store(b, _np(p[sl_d.long()]), np.arange(n), hrows2))
    for p, b in zip(pools, before):
        assert np.array_equal(_np(p[untouched]), b)


def test_prefetched_prefix_attends_like_resident():
    # a request's cached prefix is written back to the host tier, its slots are
    # reused, and the prefix is prefetched into other slots before the next
    # extend: the extend over the prefetched rows equals the one over the
    # resident rows bit for bit (the prefill kernel's result depends on the
    # values only, not on the slots)
    from prefix_shared_paged_amd import extend_attn
    Hq, Hkv, D, P, E, S, n_host = 32, 8, 128, 300, 40, 8192, 1000
    rng = np.random.default_rng(21)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    rnd = lambda *shape: (torch.randn(shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    kp, vp = rnd(S, Hkv, D), rnd(S, Hkv, D)
    q, k_new, v_new = rnd(E, Hq, D), rnd(E, Hkv, D), rnd(E, Hkv, D)
    perm = rng.permutation(S)
    s1, s_new, s2 = perm[:P], perm[P:P + E], perm[P + E:2 * P + E]
    args = lambda slots: (_dev(np.concatenate([slots, s_new])[None], torch.int32), _dev([0], torch.int32),
                          _dev([P], torch.int32), _dev([0, E], torch.int64))
    o_ref = extend_attn(q, kp, vp, *args(s1), E, k_new=k_new, v_new=v_new)
    host_k = torch.zeros((n_host, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.zeros((n_host, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    hrows = _dev(rng.permutation(n_host)[:P], torch.int64)
    sp.hicache_write_back(kp, vp, _dev(s1, torch.int32), hrows, host_k, host_v)
    kp[_dev(s1, torch.int64)] = 0
    vp[_dev(s1, torch.int64)] = 0
    sp.hicache_prefetch(host_k, host_v, hrows, _dev(s2, torch.int32), kp, vp)
    o2 = extend_attn(q, kp, vp, *args(s2), E, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o2)
