"""Extend attention over seeded random shapes (GPU, through the C ABI).

Head counts, head dims, groups, cached prefix lengths and new-token counts
are drawn from fixed seeds: half the seeds are prefill-like (up to 600 new
tokens per request, some requests none), half verify-like (1-4 new tokens
per request, which takes the split-K small-q path when q_len x Hq/Hkv <= 16).
Sampled rows of every request (its first and last new token among them) are
checked against the fp64 oracle (max |o - r| <= 2e-2, LSE within 1e-3), and
the req_to_token rows bit-exactly against the brute-force pool."""
import numpy as np
import pytest

import workloads as W
from scenarios import GroupCase, bf16_err, oracle_extend, run_extend

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3
SHAPES = [(32, 8, 128), (16, 4, 128), (8, 2, 128), (16, 16, 128), (16, 4, 64), (8, 8, 64), (64, 8, 128),
          (8, 1, 128), (4, 4, 128)]


def _case(seed):
    rng = np.random.default_rng(8000 + seed)
    Hq, Hkv, D = SHAPES[int(rng.integers(len(SHAPES)))]
    G = int(rng.integers(1, 5))
    members = rng.integers(1, 6, size=G)
    prefixes = rng.integers(0, 3000, size=G).astype(np.int64)
    if rng.random() < 0.4:
        prefixes[int(rng.integers(G))] = 0
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    B = len(grp)
    if seed % 2:
        E = rng.integers(1, 5, size=B).astype(np.int64)
    else:
        E = rng.integers(0, 600, size=B).astype(np.int64)
        E[int(rng.integers(B))] = max(1, int(E.max()))
    spec = W.Spec("random_extend", "bf16", Hq, Hkv, D, 1, 1 << 16, 0.5, 9500 + seed)
    ctx = np.array([prefixes[g] for g in grp], np.int64) + E
    return W.GroupWorkload(spec, prefixes, grp, sib, ctx), E, rng


@pytest.mark.parametrize("seed", range(8))
def test_extend_random_shapes(seed):
    wl, E, rng = _case(seed)
    case = GroupCase(wl)
    res = run_extend(case, E)
    case.check_r2t()
    sample = []
    for r in range(wl.B):
        if E[r] == 0:
            continue
        ii = {0, int(E[r]) - 1} | set(rng.integers(0, E[r], size=min(10, int(E[r]))).tolist())
        sample += [(r, int(i)) for i in sorted(ii)]
    idx, O, LSE = oracle_extend(case, res, rows_sample=sample)
    err = bf16_err(res["o"][idx], O)
    lerr = float(np.max(np.abs(res["lse"][idx] - LSE)))
    s = wl.spec
    print(f"random extend seed={seed} Hq={s.Hq} Hkv={s.Hkv} D={s.D} B={wl.B} max E={int(E.max())}: "
          f"{len(idx)} rows, max abs err {err:.3e}, lse err {lerr:.2e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL
