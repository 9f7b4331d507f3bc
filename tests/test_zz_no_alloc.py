"""The allocation-free cascade decode (sgl_cascade_decode_attn_static)
against the workspace entry point (sgl_cascade_decode_attn), through the C
ABI: two calls in a row on the same GPU, the second with a smaller input, so
the static scratch holds the first call's states when the second runs.  Both
entry points run the same kernels with the same splits, so their outputs
must agree bit for bit; the outputs are also checked against the fp64 oracle
on sampled requests (max |o - r| <= 2e-2, LSE within 1e-3).  A call whose
split states exceed the static scratch fails with SGL_ERR_WORKSPACE before
anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
import prefix_shared_paged_amd as sp
from scenarios import GroupCase, bf16_err, dev, dev_i, oracle_decode

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3


def _case(seed, G, per_group, p_hi, l_hi, wl=None, L=None):
    if wl is None:
        wl = W.decode(seed=seed, G=G, per_group=per_group, p_lo=64, p_hi=p_hi, l_lo=p_hi // 2, l_hi=l_hi,
                      num_slots=1 << 20)
    case = GroupCase(wl)
    L = wl.ctx_len.copy() if L is None else L
    P = np.array([wl.prefix_len[wl.grp[r]] for r in range(wl.B)], np.int64)
    rows = case.admit_requests(L - P)
    case.cache.append(rows, L - P)
    for st, n in zip(rows, L - P):
        case.mirror.append(st.row, int(n))
    for r, st in enumerate(rows):
        n_hist = int(L[r] - P[r] - 1)
        if n_hist > 0:
            Ks, Vs = case.suffix_kv(r)
            case.cache.store(dev(Ks[:n_hist], "bf16"), dev(Vs[:n_hist], "bf16"), st.slots[P[r]:L[r] - 1])
    kn = np.stack([case.suffix_kv(r)[0][L[r] - P[r] - 1] for r in range(wl.B)])
    vn = np.stack([case.suffix_kv(r)[1][L[r] - P[r] - 1] for r in range(wl.B)])
    q = np.stack([wl.queries(r, 1)[0] for r in range(wl.B)])
    gptr = np.zeros(wl.G + 1, np.int32)
    gptr[1:] = np.cumsum(np.bincount(wl.grp, minlength=wl.G))
    c = case.cache
    args = (dev(q, "bf16"), c.k_pool, c.v_pool, c.r2t, c.rows_tensor(rows), dev_i(L), dev_i(gptr),
            dev_i(wl.prefix_len), int(L.max()), int(np.diff(gptr).max()), int(wl.prefix_len.max()))
    return case, dict(q=q, L=L, P=P), args, (dev(kn, "bf16"), dev(vn, "bf16"))


def _run_both(case, res, args, kv):
    wl = case.wl
    B, Hq = wl.B, wl.spec.Hq
    l1 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    # the workspace entry point stores the current token; the static one
    # then attends over the same pool
    o1 = sp.cascade_decode_attn(*args, k_new=kv[0], v_new=kv[1], lse=l1)
    o2 = sp.cascade_decode_attn_static(*args, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), \
        f"static vs workspace entry: max |do| {float((o1.float() - o2.float()).abs().max()):.3e}"
    sample = sorted(set(np.random.default_rng(0).choice(B, min(B, 24), replace=False).tolist() + [B - 1]))
    reqs, O, LSE = oracle_decode(case, res, reqs=sample)
    err = bf16_err(o2.float().cpu().numpy()[reqs], O)
    lerr = float(np.max(np.abs(l2.cpu().numpy()[reqs] - LSE)))
    print(f"static cascade B={B}: max abs err {err:.3e}, lse err {lerr:.2e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL


def test_static_scratch_two_calls_second_smaller():
    assert sp.static_scratch_bytes() == 128 << 20
    case, res, args, kv = _case(seed=3, G=8, per_group=16, p_hi=3000, l_hi=5000)
    _run_both(case, res, args, kv)
    case2, res2, args2, kv2 = _case(seed=4, G=3, per_group=5, p_hi=700, l_hi=1500)
    _run_both(case2, res2, args2, kv2)


def test_static_scratch_fork_two_launches():
    # the fork shape (prefix items longer than the suffix items) runs the two
    # stages in two launches, the first also computing the suffix starts
    wl = W.fork(seed=5, G=16, branches=8, prompt=4096, max_suffix=40, num_slots=1 << 17)
    L = np.full(wl.B, 4096 + 40, np.int64)
    case, res, args, kv = _case(5, 0, 0, 0, 0, wl=wl, L=L)
    _run_both(case, res, args, kv)


def test_static_scratch_rejects_oversized_call():
    # 1024 requests over contexts of up to 32768 keys: their split states
    # (>= 2 GB) cannot fit the 128 MiB scratch; the call fails before launching
    B, Hq, Hkv, D, stride = 1024, 32, 8, 128, 32768
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    r2t = torch.zeros((B, stride), dtype=torch.int32, device="cuda")
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    seq = torch.full((B,), stride, dtype=torch.int32, device="cuda")
    gptr = torch.tensor([0, B], dtype=torch.int32, device="cuda")
    gpl = torch.tensor([8], dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, D), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sp.SglError) as e:
        sp.cascade_decode_attn_static(q, pool, pool, r2t, rows, seq, gptr, gpl, stride, B, 8, o=o)
    assert e.value.status == sp.SGL_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
