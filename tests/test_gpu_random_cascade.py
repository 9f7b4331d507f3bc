"""Cascade decode over seeded random shapes (GPU, through the C ABI).

Head counts, head dims, group counts and sizes, prefix and suffix lengths are
drawn from fixed seeds; the pools hold bf16 values or FP8 (e4m3fn) codes; each
call stores its requests' current tokens itself.  Every request's output and
log-sum-exp are checked against the fp64 oracle (max |o - r| <= 2e-2, LSE
within 1e-3) and the stored rows against the inputs (bf16 values exactly, FP8
codes equal to oracle.fp8.quantize), so the call's paths -- one grid or two
launches, the store carried by the prefix-stage launch, suffix grids sized
below the longest suffix, the merge's one-round and multi-pass forms -- meet
the oracle on shapes that no other test fixes."""
import numpy as np
import pytest
import torch

import oracle.fp8 as F8
import workloads as W
from scenarios import GroupCase, bf16_err, oracle_decode, run_decode

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3
SHAPES = [(32, 8, 128), (16, 4, 128), (8, 2, 128), (16, 16, 128), (16, 4, 64), (8, 8, 64), (64, 8, 128),
          (8, 1, 128)]


def _workload(seed):
    rng = np.random.default_rng(7000 + seed)
    Hq, Hkv, D = SHAPES[int(rng.integers(len(SHAPES)))]
    G = int(rng.integers(1, 6))
    members = rng.integers(1, 9, size=G)
    prefixes = rng.integers(0, 3000, size=G).astype(np.int64)
    if rng.random() < 0.4:
        prefixes[int(rng.integers(G))] = 0               # a group with no shared prefix
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    long_tail = rng.random() < 0.5                        # some suffixes far longer than the rest
    L = np.array([prefixes[g] + (int(rng.integers(1, 4000)) if long_tail and rng.random() < 0.2
                                 else int(rng.integers(1, 300))) for g in grp], np.int64)
    spec = W.Spec("random_cascade", "bf16", Hq, Hkv, D, 1, 1 << 17, 0.5, 9000 + seed)
    return W.GroupWorkload(spec, prefixes, grp, sib, L)


def _check_current_rows(case, res):
    """The pool rows at every request's current position hold the token the
    call stored: the bf16 values, or the oracle's FP8 codes of them."""
    cur = [int(st.slots[int(res["L"][r]) - 1]) for r, st in enumerate(case.rows)]
    idx = torch.tensor(cur, dtype=torch.long, device="cuda")
    kg, vg = case.cache.k_pool[idx], case.cache.v_pool[idx]
    kg = (kg.cpu().numpy() if case.fp8 else kg.float().cpu().numpy())
    vg = (vg.cpu().numpy() if case.fp8 else vg.float().cpu().numpy())
    for r in range(len(cur)):
        n = int(res["L"][r] - res["P"][r])
        Ks, Vs = case.suffix_kv(r)
        if case.fp8:
            ks, vs = case.kv_scale
            np.testing.assert_array_equal(kg[r], F8.quantize(Ks[n - 1:n], ks)[0])
            np.testing.assert_array_equal(vg[r], F8.quantize(Vs[n - 1:n], vs)[0])
        else:
            np.testing.assert_array_equal(kg[r], Ks[n - 1])
            np.testing.assert_array_equal(vg[r], Vs[n - 1])


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed", range(8))
def test_cascade_random_shapes(seed, fp8):
    wl = _workload(seed)
    case = GroupCase(wl, fp8=fp8)
    res = run_decode(case, wl.ctx_len.copy(), cascade=True)
    case.check_r2t()
    _check_current_rows(case, res)
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    s = wl.spec
    print(f"random cascade seed={seed} fp8={fp8} Hq={s.Hq} Hkv={s.Hkv} D={s.D} B={wl.B} G={wl.G}: "
          f"max abs err {err:.3e}, lse err {lerr:.2e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL


# ---------------------------------------------------------------------------
# balanced suffix stage: bf16 calls whose suffixes reach 1024 keys or more
# (max_seq_len - max_prefix_len >= 1024) lay the suffixes end to end and give
# every workgroup an equal run; runs cross requests, long suffixes span many
# runs (the merge then has more parts than its one-round form holds), and
# one-key suffixes sit between long ones
# ---------------------------------------------------------------------------
def _balanced_workload(seed, Hq, Hkv, D, n_req=48):
    rng = np.random.default_rng(8100 + seed)
    prefixes = np.array([0, 1, 300, 1000, 2047, 64], np.int64)
    members = np.full(len(prefixes), n_req // len(prefixes))
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    suf = rng.integers(1, 3200, size=len(grp))
    suf[::7] = 1                                   # the current token only
    suf[3::11] = int(rng.integers(3000, 4000))     # long suffixes over many runs
    L = np.array([prefixes[g] + s for g, s in zip(grp, suf)], np.int64)
    spec = W.Spec("balanced_suffix", "bf16", Hq, Hkv, D, 1, 1 << 18, 0.5, 8200 + seed)
    return W.GroupWorkload(spec, prefixes, grp, sib, L)


@pytest.mark.parametrize("store", [True, False])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 128), (16, 16, 128), (16, 4, 64)])
def test_cascade_balanced_suffix(Hq, Hkv, D, store):
    wl = _balanced_workload(Hkv + D, Hq, Hkv, D)
    assert int(wl.ctx_len.max() - wl.prefix_len.max()) >= 1024
    case = GroupCase(wl)
    # store: the cascade call stores the current tokens; else the flat call
    # stores them and the cascade call (o_c) reads them from the pool
    res = run_decode(case, wl.ctx_len.copy(), cascade=True, both=not store)
    case.check_r2t()
    _check_current_rows(case, res)
    reqs, O, LSE = oracle_decode(case, res)
    o, l = (res["o"], res["lse"]) if store else (res["o_c"], res["lse_c"])
    err = bf16_err(o[reqs], O)
    lerr = float(np.max(np.abs(l[reqs] - LSE)))
    print(f"balanced suffix Hq={Hq} Hkv={Hkv} D={D} store={store} B={wl.B}: max abs err {err:.3e}, "
          f"lse err {lerr:.2e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL
