"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (stated by the target of this work): fp32 inputs -> max over
(row, head) of ||o - r||_inf / ||r||_inf <= 1e-5; bf16 inputs -> max |o - r|
<= 2e-2 with r computed in fp64 from the same bf16 values.  req_to_token rows
and match lengths are compared bit-exactly with the brute-force model.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from prefix_shared_paged_amd import decode_attn, extend_attn
from scenarios import (GroupCase, bf16_err, dev, dev_i, f32_rel_err, late_rounds_workload, many_rounds_workload,
                       oracle_decode, oracle_extend, run_decode, run_extend)

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5
# Log-sum-exp of the scaled scores (natural log), every bf16 kernel, extend
# and decode alike.  The scores and the row sums are fp32 (only the weights
# entering the PV product are rounded to bf16), so the kernels' value differs
# from the exact one by fp32 rounding alone: the score sums over D <= 128
# products move a scaled score by at most ~1.5e-4 for the 8x-wide "peaky"
# queries (2e-5 for the others), and the row sum, a 16-term tree per key tile
# added tile after tile, is off by at most (tiles + 5) * 2^-24 relative
# (< 5e-5 at 20k keys).  The fixed tolerance sits above that worst case; a
# key missed or counted twice moves the value by that key's share of the row
# sum, which the peaky variants make large.
LSE_TOL = 1e-3


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# tiny fp32 workload: setup extend (P = 0), extend step, decode step
# ---------------------------------------------------------------------------
def test_tiny_fp32_extend_then_decode():
    wl = W.tiny(seed=0)
    s = wl.spec
    case = GroupCase(wl, creator_extend=True)
    # the setup extend of the shared prefix with nothing cached = dense causal attention
    g, q0, o0 = case.creator_out[0]
    K, V = case.prefix_kv[0]
    O, _, _, _ = oracle.attention([K], [V], np.zeros(64), np.arange(64), q0, s.Hq, s.Hkv)
    err = f32_rel_err(o0, O)
    _print("tiny creator extend rel err", err)
    assert err <= F32_TOL
    # step 1: 4 requests match 64 and extend 16 each
    E = np.full(wl.B, 16, np.int64)
    res = run_extend(case, E)
    case.check_r2t()
    idx, O, LSE = oracle_extend(case, res)
    err = f32_rel_err(res["o"][idx], O)
    _print("tiny extend rel err", err)
    assert err <= F32_TOL
    assert np.max(np.abs(res["lse"][idx] - LSE)) < 1e-4
    # step 2: the same requests decode one token each at position 80 (L = 81)
    rows = case.rows
    case.cache.append(rows, [1] * wl.B)
    for st in rows:
        case.mirror.append(st.row, 1)
    case.check_r2t()
    kn = np.stack([case.suffix_kv(r)[0][16] for r in range(wl.B)])
    vn = np.stack([case.suffix_kv(r)[1][16] for r in range(wl.B)])
    q = np.stack([wl.queries(r, 1, step=1)[0] for r in range(wl.B)])
    L = np.full(wl.B, 81, np.int32)
    o = decode_attn(dev(q, "f32"), case.cache.k_pool, case.cache.v_pool, case.cache.r2t,
                    case.cache.rows_tensor(rows), dev_i(L), 81, k_new=dev(kn, "f32"), v_new=dev(vn, "f32"))
    from prefix_shared_paged_amd import cascade_decode_attn
    oc = cascade_decode_attn(dev(q, "f32"), case.cache.k_pool, case.cache.v_pool, case.cache.r2t,
                             case.cache.rows_tensor(rows), dev_i(L), dev_i([0, wl.B]), dev_i([64]), 81,
                             wl.B, 64)
    torch.cuda.synchronize()
    for r in range(wl.B):
        Kr, Vr = case.logical_kv(r, 17)
        Or, _, _, _ = oracle.attention([Kr], [Vr], [0], [80], q[r][None], s.Hq, s.Hkv)
        e1 = f32_rel_err(o[r].cpu().numpy()[None], Or)
        e2 = f32_rel_err(oc[r].cpu().numpy()[None], Or)
        _print("tiny decode rel err", r, e1, e2)
        assert e1 <= F32_TOL and e2 <= F32_TOL


# ---------------------------------------------------------------------------
# extend: small ragged cases (several tiles, ragged tails, GQA widths, D 64)
# ---------------------------------------------------------------------------
def _small_extend_workload(seed, Hq, Hkv, D, prefixes, members, dtype="bf16", q_scale=1.0):
    spec = W.Spec("small", dtype, Hq, Hkv, D, 1, 1 << 14, 0.5 if dtype == "bf16" else 1.0, seed,
                  extra={"q_scale": q_scale})
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    ctx = np.array([prefixes[g] + 300 for g in grp], np.int64)
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, ctx)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 64), (16, 2, 128), (64, 8, 128), (8, 4, 64)])
def test_extend_small_ragged(Hq, Hkv, D):
    wl = _small_extend_workload(1, Hq, Hkv, D, prefixes=[0, 37, 200], members=[2, 2, 2])
    case = GroupCase(wl)
    E = np.array([1, 130, 77, 0, 33, 257], np.int64)
    res = run_extend(case, E)
    case.check_r2t()
    idx, O, LSE = oracle_extend(case, res)
    err = bf16_err(res["o"][idx], O)
    lerr = float(np.max(np.abs(res["lse"][idx] - LSE)))
    _print(f"extend small Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64)])
def test_extend_small_ragged_peaky(Hq, Hkv, D):
    # queries 8x wider (N(0,1) x 4): scores spread over a few units, so the
    # softmax concentrates on few keys and a key missed or counted twice
    # shows in o
    wl = _small_extend_workload(11, Hq, Hkv, D, prefixes=[0, 37, 200], members=[2, 2, 2], q_scale=8.0)
    case = GroupCase(wl)
    E = np.array([1, 130, 77, 0, 33, 257], np.int64)
    res = run_extend(case, E)
    idx, O, LSE = oracle_extend(case, res)
    err = bf16_err(res["o"][idx], O)
    lerr = float(np.max(np.abs(res["lse"][idx] - LSE)))
    _print(f"extend peaky Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


def test_extend_fp32_small_ragged():
    wl = _small_extend_workload(2, 8, 2, 128, prefixes=[5, 64], members=[2, 1], dtype="f32")
    case = GroupCase(wl)
    E = np.array([70, 1, 129], np.int64)
    res = run_extend(case, E)
    idx, O, _ = oracle_extend(case, res)
    err = f32_rel_err(res["o"][idx], O)
    _print("extend fp32 small rel err", err)
    assert err <= F32_TOL


# ---------------------------------------------------------------------------
# extend at full size: 64 requests x 256 new over a cached 2048-token prefix
# ---------------------------------------------------------------------------
def test_extend_full_size_sampled():
    wl = W.extend(seed=0)
    case = GroupCase(wl)
    E = np.full(wl.B, 256, np.int64)
    res = run_extend(case, E)
    case.check_r2t()
    rng = np.random.default_rng(5)
    sample = [(r, i) for r in range(wl.B) for i in sorted({0, 1, 31, 32, 127, 255, int(rng.integers(256))})]
    idx, O, LSE = oracle_extend(case, res, rows_sample=sample)
    err = bf16_err(res["o"][idx], O)
    lerr = float(np.max(np.abs(res["lse"][idx] - LSE)))
    _print(f"extend full-size sampled {len(idx)} rows: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL
    # every output is finite
    assert np.isfinite(res["o"]).all()


# ---------------------------------------------------------------------------
# GPU invariants
# ---------------------------------------------------------------------------
def _direct_extend(order, P, E, seed=3, Hq=32, Hkv=8, D=128, slots=4096):
    """One request, logical K/V of P + E tokens; the first P stored as cached prefix."""
    spec = W.Spec("inv", "bf16", Hq, Hkv, D, 1, slots, 0.5, seed)
    K = W.values(spec, (P + E, Hkv, D), 1)
    V = W.values(spec, (P + E, Hkv, D), 2)
    Q = W.values(spec, (P + E, Hq, D), 3)
    from prefix_shared_paged_amd.paged_cache import PagedKVCache
    c = PagedKVCache(slots, 1, Hkv, D, torch.bfloat16, 2, P + E + 1, order)
    [st] = c.admit([np.arange(P + E, dtype=np.int32) + 1])
    c.append([st], [P + E])
    c.store(dev(K[:P], "bf16"), dev(V[:P], "bf16"), st.slots[:P])
    o = extend_attn(dev(Q[P:], "bf16"), c.k_pool, c.v_pool, c.r2t, c.rows_tensor([st]), dev_i([P]),
                    dev_i([0, E], torch.int64), E, k_new=dev(K[P:], "bf16"), v_new=dev(V[P:], "bf16"))
    torch.cuda.synchronize()
    return o.cpu()


def test_prefix_reuse_equals_recompute_bitwise():
    # prefill kernel: rows P.. of extend(P cached, E new) == the same rows of
    # extend(0 cached, P+E new), bit for bit (a row's result depends only on
    # its keys, not on where the cached part ends)
    order = np.random.default_rng(0).permutation(4096).astype(np.int32)
    for P, E in [(100, 50), (64, 64), (1, 200), (290, 10)]:
        a = _direct_extend(order, P, E)
        b = _direct_extend(order, 0, P + E)
        assert torch.equal(a, b[P:]), (P, E)
    # one new token (4 query rows per KV head) takes the split-K small-q path,
    # whose splits follow the context length and whose merge rounds
    # differently: equal to the recomputation within the bf16 tolerance
    a = _direct_extend(order, 300, 1)
    b = _direct_extend(order, 0, 301)
    assert float((a.float() - b[300:].float()).abs().max()) <= BF16_TOL


def test_slot_permutation_invariance_bitwise():
    o1 = _direct_extend(np.random.default_rng(1).permutation(4096).astype(np.int32), 150, 90)
    o2 = _direct_extend(np.random.default_rng(2).permutation(4096).astype(np.int32), 150, 90)
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------------------
# long contexts and very large pools
# ---------------------------------------------------------------------------
def _pool_extend_case(spec, P_list, E_list, slots_of, num_slots, seed):
    """Requests with prefixes P_list and new tokens E_list whose K/V rows live at
    slots_of(r, n) in pools of num_slots rows (only those rows are written)."""
    Hq, Hkv, D = spec.Hq, spec.Hkv, spec.D
    kp = torch.zeros((num_slots, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((num_slots, Hkv, D), dtype=torch.bfloat16, device="cuda")
    stride = max(p + e for p, e in zip(P_list, E_list)) + 3
    r2t = torch.full((len(P_list), stride), -1, dtype=torch.int32, device="cuda")
    Ks, Vs, Qs = [], [], []
    for r, (P, E) in enumerate(zip(P_list, E_list)):
        K = W.values(spec, (P + E, Hkv, D), 10 + r)
        V = W.values(spec, (P + E, Hkv, D), 20 + r)
        Q = W.values(spec, (E, Hq, D), 30 + r) * np.float32(spec.extra.get("q_scale", 1.0))
        sl = slots_of(r, P + E)
        assert len(set(sl.tolist())) == P + E and sl.min() >= 0 and sl.max() < num_slots
        idx = torch.as_tensor(sl, dtype=torch.int64, device="cuda")
        kp[idx] = dev(K, "bf16")
        vp[idx] = dev(V, "bf16")
        r2t[r, :P + E] = dev_i(sl)
        Ks.append(K), Vs.append(V), Qs.append(Q)
    return kp, vp, r2t, Ks, Vs, Qs


def _check_extend_rows(o, Ks, Vs, Qs, P_list, E_list, spec, rng, n_rows=6):
    q_off = np.concatenate([[0], np.cumsum(E_list)])
    worst = 0.0
    for r, (P, E) in enumerate(zip(P_list, E_list)):
        rows = sorted(set([0, E - 1] + rng.integers(0, E, n_rows).tolist()))
        want, _, _, _ = oracle.attention([Ks[r]], [Vs[r]], np.zeros(len(rows)), P + np.array(rows),
                                         Qs[r][rows], spec.Hq, spec.Hkv)
        got = o[q_off[r] + np.array(rows)].float().cpu().numpy()
        worst = max(worst, bf16_err(got, want))
    return worst


def _check_last_row_lse(lse, Ks, Vs, Qs, P_list, E_list, spec):
    """The log-sum-exp of the last new token of each request, within LSE_TOL."""
    Hq, Hkv = spec.Hq, spec.Hkv
    q_off = np.concatenate([[0], np.cumsum(E_list)])
    worst = 0.0
    for r, (P, E) in enumerate(zip(P_list, E_list)):
        _, _, _, LSE = oracle.attention([Ks[r]], [Vs[r]], [0], [P + E - 1], Qs[r][E - 1:E], Hq, Hkv)
        worst = max(worst, float(np.max(np.abs(lse[q_off[r] + E - 1].cpu().numpy() - LSE[0]))))
    _print(f"  last-row lse err {worst:.2e}")
    assert worst <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64)])
def test_extend_long_context(Hq, Hkv, D):
    # contexts of 9000+ keys: the kernel's LDS slot table (4096 keys) is
    # refilled several times while the keys stream through
    spec = W.Spec("long", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, 5)
    P_list, E_list = [9000, 4100, 33], [70, 129, 1]
    perm = np.random.default_rng(5).permutation(1 << 15).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(np.array(P_list) + np.array(E_list))])
    kp, vp, r2t, Ks, Vs, Qs = _pool_extend_case(spec, P_list, E_list, lambda r, n: perm[offs[r]:offs[r] + n],
                                                1 << 15, 5)
    q = dev(np.concatenate(Qs), "bf16")
    lse = torch.empty((sum(E_list), Hq), dtype=torch.float32, device="cuda")
    o = extend_attn(q, kp, vp, r2t, dev_i(range(len(P_list))), dev_i(P_list),
                    dev_i(np.concatenate([[0], np.cumsum(E_list)]), torch.int64), max(E_list), lse=lse)
    torch.cuda.synchronize()
    err = _check_extend_rows(o, Ks, Vs, Qs, P_list, E_list, spec, np.random.default_rng(0))
    _print(f"long-context extend Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}")
    assert err <= BF16_TOL
    _check_last_row_lse(lse, Ks, Vs, Qs, P_list, E_list, spec)


@pytest.mark.parametrize("P_list,E_list,qs", [([20000], [512], 1.0), ([12000, 3, 8191], [100, 17, 2], 1.0),
                                              ([12000, 3, 8191], [100, 17, 2], 8.0)])
def test_extend_key_splits(P_list, E_list, qs):
    # grids of a few requests over long contexts (the last rounds of chunked
    # prefill): each workgroup's keys are cut into 4096-key splits and merged;
    # contexts end inside, on and just past split boundaries
    spec = W.Spec("keysplit", "bf16", 64, 8, 128, 1, 1 << 16, 0.5, 9, extra={"q_scale": qs})
    perm = np.random.default_rng(9).permutation(1 << 16).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(np.array(P_list) + np.array(E_list))])
    kp, vp, r2t, Ks, Vs, Qs = _pool_extend_case(spec, P_list, E_list, lambda r, n: perm[offs[r]:offs[r] + n],
                                                1 << 16, 9)
    from prefix_shared_paged_amd import extend_workspace_size
    assert extend_workspace_size(len(P_list), sum(E_list), max(E_list), r2t.shape[1], 64, 8, 128) > 0
    q = dev(np.concatenate(Qs), "bf16")
    lse = torch.empty((sum(E_list), 64), dtype=torch.float32, device="cuda")
    o = extend_attn(q, kp, vp, r2t, dev_i(range(len(P_list))), dev_i(P_list),
                    dev_i(np.concatenate([[0], np.cumsum(E_list)]), torch.int64), max(E_list), lse=lse)
    torch.cuda.synchronize()
    err = _check_extend_rows(o, Ks, Vs, Qs, P_list, E_list, spec, np.random.default_rng(1))
    _print(f"key-split extend P={P_list} E={E_list}: max abs err {err:.3e}")
    assert err <= BF16_TOL
    _check_last_row_lse(lse, Ks, Vs, Qs, P_list, E_list, spec)


def test_pool_over_4gib_extend_and_decode():
    # a pool whose byte size exceeds 2^32 per K/V view, with rows above the
    # 4 GiB mark: the kernels must take 64-bit row offsets
    spec = W.Spec("bigpool", "bf16", 32, 8, 128, 1, 1, 0.5, 6)
    num_slots = (1 << 21) + 4096                    # 2048 bytes per slot -> 4.3 GB per pool
    P_list, E_list = [1500, 700], [90, 33]
    rng = np.random.default_rng(6)
    high = (1 << 21) - 2048 + rng.permutation(6144)  # straddles the 2^32-byte mark

    def slots_of(r, n):
        return np.concatenate([high[r * 3000:r * 3000 + n // 2], 17 + 5000 * r + np.arange(n - n // 2)]).astype(np.int32)

    kp, vp, r2t, Ks, Vs, Qs = _pool_extend_case(spec, P_list, E_list, slots_of, num_slots, 6)
    q = dev(np.concatenate(Qs), "bf16")
    o = extend_attn(q, kp, vp, r2t, dev_i([0, 1]), dev_i(P_list),
                    dev_i(np.concatenate([[0], np.cumsum(E_list)]), torch.int64), max(E_list))
    torch.cuda.synchronize()
    err = _check_extend_rows(o, Ks, Vs, Qs, P_list, E_list, spec, rng)
    # decode of the last token of each request over the same pool
    L = [p + e for p, e in zip(P_list, E_list)]
    qd = dev(np.stack([Qs[r][-1] for r in range(2)]), "bf16")
    od = decode_attn(qd, kp, vp, r2t, dev_i([0, 1]), dev_i(L), max(L))
    torch.cuda.synchronize()
    want, _, _, _ = oracle.attention(Ks, Vs, np.arange(2), np.array(L) - 1, np.stack([Qs[r][-1] for r in range(2)]),
                                     spec.Hq, spec.Hkv)
    derr = bf16_err(od.float().cpu().numpy(), want)
    _print(f"pool over 4 GiB: extend max abs err {err:.3e}, decode {derr:.3e}")
    del kp, vp
    torch.cuda.empty_cache()
    assert err <= BF16_TOL and derr <= BF16_TOL


# ---------------------------------------------------------------------------
# decode and cascade decode
# ---------------------------------------------------------------------------
def _small_decode_workload(seed, Hq=32, Hkv=8, D=128, q_scale=1.0, dtype="bf16"):
    spec = W.Spec("small_dec", dtype, Hq, Hkv, D, 1, 1 << 15, 0.5 if dtype == "bf16" else 1.0, seed,
                  extra={"q_scale": q_scale})
    members = [1, 3, 5, 16]
    prefixes = [0, 1, 300, 256]
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    rng = np.random.default_rng(seed)
    L = np.array([rng.integers(prefixes[g] + 1, 1300) for g in grp], np.int64)
    L[1] = 2      # prefix 1 + current token
    L[4] = 301    # suffix is only the current token
    L[9] = 257
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, L)


@pytest.mark.parametrize("cascade", [False, True])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 128), (8, 8, 64), (16, 4, 128), (32, 16, 128)])
def test_decode_small(cascade, Hq, Hkv, D):
    # the 16-member group gives 16 * Hq/Hkv query rows per KV head: 128 rows
    # (two 64-row waves) for Hq/Hkv = 8; 4 and 16 KV heads at D 128 put one
    # and four groups of 4 KV heads in the cascade's whole-row suffix items
    wl = _small_decode_workload(7, Hq, Hkv, D)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"decode small cascade={cascade} Hq={Hq}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("cascade", [False, True])
@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 64), (16, 4, 128)])
def test_decode_fp32_small(cascade, Hq, Hkv, D):
    # the fp32 kernels walk keys in blocks of 64: lengths on and beside the
    # block edges, suffixes of one and 64 keys, a prefix of one key
    wl = _small_decode_workload(9, Hq, Hkv, D, dtype="f32")
    L = wl.ctx_len.copy()
    L[2], L[3], L[5], L[6], L[7] = 64, 65, 364, 365, 300 + 128
    L[10], L[11], L[12] = 256 + 1, 256 + 63, 256 + 64
    wl = W.GroupWorkload(wl.spec, wl.prefix_len, wl.grp, wl.sib, L)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    err = f32_rel_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"decode fp32 small cascade={cascade} Hq={Hq} D={D}: max rel err {err:.3e}, lse err {lerr:.2e}")
    assert err <= F32_TOL and lerr <= 1e-4


@pytest.mark.parametrize("cascade", [False, True])
def test_decode_small_peaky(cascade):
    # queries 8x wider (see test_extend_small_ragged_peaky)
    wl = _small_decode_workload(17, 32, 8, 128, q_scale=8.0)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade)
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"decode peaky cascade={cascade}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


def _split_edge_workload(seed, Hq, Hkv, D):
    """Groups whose prefix and context lengths sit on and next to the
    kernels' split (1024 keys) and tile (16 keys) boundaries, with group sizes
    that leave partial 16-row blocks and idle waves in the prefix stage."""
    spec = W.Spec("split_edges", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, seed)
    members = [1, 2, 5, 9]
    prefixes = [1024, 16, 1023, 17]
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    L = np.array([1025,                                  # suffix = current token only
                  17, 2048,                              # one-token suffix; split-aligned context
                  1024, 1025, 2047, 2049, 3072,          # contexts around 1024-key splits
                  18, 33, 1040, 1041, 2065, 3000, 3090, 4096, 4097], np.int64)
    assert len(L) == len(grp)
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, L)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 64), (16, 2, 64), (8, 1, 128)])
def test_decode_split_and_group_edges(Hq, Hkv, D):
    # (16, 4, 64): 36 rows per KV head in the 9-member group -> 3 row blocks
    # on 2-wave workgroups; (16, 2, 64): 72 rows; (8, 1, 128): one KV head
    wl = _split_edge_workload(11, Hq, Hkv, D)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode split edges {tag} Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 128), (16, 4, 64)])
def test_cascade_late_suffix_rounds(Hq, Hkv, D):
    # (32, 8, 128): one grid, the long suffixes' later rounds after the prefix
    # items; (16, 2, 128) and (16, 4, 64): two launches, the suffix grid sized
    # for the short suffixes and its workgroups running the later rounds
    wl = late_rounds_workload(29, Hq, Hkv, D)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode late suffix rounds {tag} Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 128), (16, 4, 64)])
def test_cascade_many_later_rounds(Hq, Hkv, D):
    wl = many_rounds_workload(37, Hq, Hkv, D)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade=True)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"cascade many later rounds Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


def test_decode_full_size_flat_and_cascade():
    wl = W.decode(seed=0)
    case = GroupCase(wl)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    case.check_r2t()
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode full {tag}: {len(reqs)} requests, max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("s", [1, 2, 64, 255, 256, 512])
def test_fork_cascade(s):
    wl = W.fork(seed=0)
    case = GroupCase(wl)
    L = np.full(wl.B, 4096 + s, np.int64)
    res = run_decode(case, L, cascade=False, both=True)
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    err_c = bf16_err(res["o_c"][reqs], O)
    _print(f"fork s={s}: flat max abs err {err:.3e}, cascade {err_c:.3e}")
    assert err <= BF16_TOL and err_c <= BF16_TOL


def _check_current_rows(case, res):
    """The pool rows at every request's current position hold the token the
    call stored (bf16 values, exactly)."""
    cur = [int(st.slots[int(res["L"][r]) - 1]) for r, st in enumerate(case.rows)]
    idx = torch.tensor(cur, dtype=torch.long, device="cuda")
    kg = case.cache.k_pool[idx].float().cpu().numpy()
    vg = case.cache.v_pool[idx].float().cpu().numpy()
    for r in range(len(cur)):
        n = int(res["L"][r] - res["P"][r])
        Ks, Vs = case.suffix_kv(r)
        np.testing.assert_array_equal(kg[r], Ks[n - 1])
        np.testing.assert_array_equal(vg[r], Vs[n - 1])


@pytest.mark.parametrize("wl_name,s", [("fork", 1), ("fork", 64), ("small_8_8_64", 0), ("small_16_2_128", 0)])
def test_cascade_stores_current_token(wl_name, s):
    # the cascade call itself stores the current tokens.  On these shapes it
    # runs its stages in two launches (the fork's prefix items are the longer
    # ones; D 64; 2 KV heads), so the store and the suffix starts run in
    # leading workgroups of the prefix-stage launch
    if wl_name == "fork":
        wl = W.fork(seed=1)
        L = np.full(wl.B, 4096 + s, np.int64)
        sample = list(range(0, wl.B, 4))
    else:
        Hq, Hkv, D = (int(x) for x in wl_name.split("_")[1:])
        wl = _small_decode_workload(23, Hq, Hkv, D)
        L = wl.ctx_len.copy()
        sample = None
    case = GroupCase(wl)
    res = run_decode(case, L, cascade=True)
    _check_current_rows(case, res)
    reqs, O, LSE = oracle_decode(case, res, reqs=sample)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"cascade with store {wl_name} s={s}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("P,E", [(12000, 100), (3000, 2)])
def test_extend_without_workspace_runs_unsplit(P, E):
    # key splits (one long request) and the small-q split-K path (2 new tokens)
    # need split-state workspace; given none, the call runs the prefill kernel
    # unsplit: the same attention within rounding
    Hq, Hkv, D, S = 32, 8, 128, 1 << 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(P + E)
    rnd = lambda *shape: (torch.randn(shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    kp, vp, q = rnd(S, Hkv, D), rnd(S, Hkv, D), rnd(E, Hq, D)
    r2t = torch.randperm(S, generator=gen, device="cuda")[:P + E].to(torch.int32)[None]
    args = (q, kp, vp, r2t, dev_i([0]), dev_i([P]), dev_i([0, E], torch.int64), E)
    l1 = torch.empty((E, Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty((E, Hq), dtype=torch.float32, device="cuda")
    o1 = extend_attn(*args, lse=l1)
    o2 = extend_attn(*args, lse=l2, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    err = float((o1.float() - o2.float()).abs().max())
    lerr = float((l1 - l2).abs().max())
    _print(f"extend P={P} E={E}: split vs unsplit max abs diff {err:.3e}, lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


def test_cascade_workspace_sized_for_larger_bounds():
    # a workspace sized for the longest suffix of a sweep serves the calls with
    # shorter suffixes, which would prefer smaller (so more) suffix splits: the
    # call fits its splits to the workspace it is given
    import prefix_shared_paged_amd as sp
    wl = W.fork(seed=0)
    P0 = int(wl.prefix_len.max())
    big = sp.cascade_workspace_size(wl.B, wl.G, P0 + 512, int(np.bincount(wl.grp).max()), P0, wl.spec.Hq,
                                    wl.spec.Hkv, wl.spec.D)
    for s in (2, 40):
        small = sp.cascade_workspace_size(wl.B, wl.G, P0 + s, int(np.bincount(wl.grp).max()), P0, wl.spec.Hq,
                                          wl.spec.Hkv, wl.spec.D)
        case = GroupCase(wl)
        L = np.full(wl.B, P0 + s, np.int64)
        ws = torch.empty(big, dtype=torch.uint8, device="cuda")
        res = run_decode(case, L, cascade=False, both=True, workspace=ws)
        reqs, O, LSE = oracle_decode(case, res)
        err_c = bf16_err(res["o_c"][reqs], O)
        _print(f"fork s={s} in a workspace for s=512 ({big} B; this call alone asks {small} B): "
               f"cascade max abs err {err_c:.3e}")
        assert err_c <= BF16_TOL


# ---------------------------------------------------------------------------
# small-q extend (a few new tokens per request over a cached context: the
# verify step of speculative decoding) -- the split-K path of sgl_extend_attn
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 128), (8, 8, 64), (16, 2, 128), (8, 4, 64)])
def test_small_q_extend_ragged(Hq, Hkv, D, q_scale=1.0):
    # one request per group, so each request has its own cached prefix; the
    # prefixes sit on and next to the 16-key tiles and the splits, and the new
    # tokens (up to the 16 query rows per KV head of the split-K path) are ragged
    g = Hq // Hkv
    emax = max(1, 16 // g)
    prefixes = [0, 1, 15, 16, 17, 300, 1023, 2000]
    spec = W.Spec("small_q", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, 7, extra={"q_scale": q_scale})
    grp = np.arange(len(prefixes), dtype=np.int64)
    wl = W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, np.zeros(len(prefixes), np.int64),
                         np.array(prefixes, np.int64) + emax)
    case = GroupCase(wl)
    E = np.array([emax, 1, min(3, emax), emax, min(2, emax), max(1, emax // 2), 5 % emax + 1, emax], np.int64)
    res = run_extend(case, E)
    case.check_r2t()
    idx, O, LSE = oracle_extend(case, res)
    err = bf16_err(res["o"][idx], O)
    lerr = float(np.max(np.abs(res["lse"][idx] - LSE)))
    _print(f"small-q extend Hq={Hq} Hkv={Hkv} D={D} E={E.tolist()}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 4, 64)])
def test_small_q_extend_peaky(Hq, Hkv, D):
    # queries 8x wider (see test_extend_small_ragged_peaky)
    test_small_q_extend_ragged(Hq, Hkv, D, q_scale=8.0)


def _direct_verify(B, Hq, Hkv, D, P, E, seed, num_slots, sample_rows):
    """Pools filled on the device from a seeded generator, request r's context
    at random distinct slots, its new tokens' K/V already stored; runs the
    extend call and returns (o, lse) with the oracle on the sampled
    (request, token) rows (all heads)."""
    import oracle
    from prefix_shared_paged_amd import extend_attn
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    kp = (torch.randn((num_slots, Hkv, D), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    vp = (torch.randn((num_slots, Hkv, D), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    L = P + E
    slots = np.random.default_rng(seed).permutation(num_slots)[:int(L.sum())].astype(np.int32)
    off = np.concatenate([[0], np.cumsum(L)])
    stride = int(L.max()) + 1
    r2t = np.full((B, stride), -1, np.int32)
    for r in range(B):
        r2t[r, :L[r]] = slots[off[r]:off[r + 1]]
    q_off = np.concatenate([[0], np.cumsum(E)]).astype(np.int64)
    q = (torch.randn((int(E.sum()), Hq, D), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    lse = torch.empty((int(E.sum()), Hq), dtype=torch.float32, device="cuda")
    o = extend_attn(q, kp, vp, dev_i(r2t), dev_i(np.arange(B)), dev_i(P), dev_i(q_off, torch.int64),
                    int(E.max()), lse=lse)
    torch.cuda.synchronize()
    o_h, lse_h, q_h = o.float().cpu().numpy(), lse.cpu().numpy(), q.float().cpu().numpy()
    errs, lerrs = [], []
    for r, i in sample_rows:
        sl = torch.from_numpy(r2t[r, :L[r]].astype(np.int64)).cuda()
        K = kp[sl].float().cpu().numpy()
        V = vp[sl].float().cpu().numpy()
        t = int(q_off[r]) + i
        Or, _, _, Lr = oracle.attention([K], [V], [0], [int(P[r]) + i], q_h[t][None], Hq, Hkv)
        errs.append(bf16_err(o_h[t][None], Or))
        lerrs.append(float(np.max(np.abs(lse_h[t] - Lr[0]))))
    return max(errs), max(lerrs)


def test_small_q_extend_slot_table_parts():
    # 128 requests x 16 KV heads: one split per request, longer than the
    # 2048-entry slot table, so the kernel refills the table within a split
    B, Hq, Hkv, D = 128, 16, 16, 64
    rng = np.random.default_rng(3)
    P = rng.integers(2040, 4300, B).astype(np.int64)
    P[:4] = [2047, 2048, 4095, 4096]
    E = rng.integers(1, 17, B).astype(np.int64)     # g = 1: up to 16 rows per KV head
    sample = [(r, i) for r in (0, 1, 2, 3, 77, 127) for i in sorted({0, int(E[r]) // 2, int(E[r]) - 1})]
    err, lerr = _direct_verify(B, Hq, Hkv, D, P, E, 11, 1 << 20, sample)
    _print(f"small-q extend, slot-table parts: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("q_len", [1, 3, 4, 16])
def test_small_q_extend_verify_shape_sampled(q_len):
    # q_len <= 4 takes the split-K path (4 q heads per KV head), 16 the prefill kernel
    # 64 requests over cached contexts ~U[2048, 8192], 32/8 heads, D 128
    B, Hq, Hkv, D = 64, 32, 8, 128
    P = np.random.default_rng(4).integers(2048, 8193, B).astype(np.int64)
    E = np.full(B, q_len, np.int64)
    sample = [(r, i) for r in (0, 31, 63) for i in sorted({0, q_len // 2, q_len - 1})]
    err, lerr = _direct_verify(B, Hq, Hkv, D, P, E, 12, 1 << 20, sample)
    _print(f"small-q extend, verify shape q_len={q_len}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL
