"""GPU parity of the FP8 (e4m3fn) KV cache, through the C ABI.

  - sgl_store_kv_fp8 and the fused store of the decode calls: the codes in the
    pools equal oracle.fp8.quantize of the same inputs, bit for bit;
  - sgl_decode_attn_fp8kv / sgl_cascade_decode_attn_fp8kv: outputs within the
    bf16 bound (max |o - r| <= 2e-2) of the fp64 oracle over the oracle's own
    codes, decoded exactly and multiplied by the per-head factors; LSE within
    1e-3 as for the bf16 decode.
"""
import numpy as np
import pytest
import torch

import oracle.fp8 as F8
import workloads as W
from prefix_shared_paged_amd import store_kv_fp8
from scenarios import GroupCase, bf16_err, late_rounds_workload, many_rounds_workload, oracle_decode, run_decode

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3


def _print(*a):
    print(*a, flush=True)


def _store_inputs(rng, n, Hkv, D, scale, dt):
    """Values spread over the code range of each head (x = y * scale with y
    ~ N(0, 60)), the exact midpoints of neighbouring codes (ties), values
    beyond the clamp, tiny negatives and zeros."""
    y = rng.standard_normal((n, Hkv, D)) * 60.0
    pos = F8.VALUES[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    flat = y.reshape(-1)
    k = min(len(flat) // 4, 4 * len(mids))
    idx = rng.choice(len(flat), k, replace=False)
    flat[idx] = np.resize(np.concatenate([mids, -mids]), k)
    flat[rng.choice(len(flat), 64, replace=False)] = rng.choice([1000.0, -1000.0, 449.0, -470.0, 0.0, -0.0,
                                                                 -1e-6, 1e-7], 64)
    x = (flat.reshape(n, Hkv, D) * scale[None, :, None]).astype(np.float32)
    if dt == "bf16":
        x = W.round_to_bf16(x)
    return x


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("Hkv,D", [(8, 128), (4, 64), (1, 128)])
def test_store_kv_fp8_codes_bit_exact(dt, Hkv, D):
    rng = np.random.default_rng(Hkv * 1000 + D + (dt == "f32"))
    S, n = 4096, 1000
    # power-of-two factors keep every midpoint exact in bf16; two general ones too
    ks = np.array([2.0 ** -5, 0.011, 2.0 ** -3, 0.3, 1.0, 2.0 ** -8, 0.07, 4.0][:Hkv], np.float32)
    vs = np.array([0.013, 2.0 ** -6, 0.5, 2.0 ** -4, 0.021, 1.0, 2.0 ** -2, 0.0009][:Hkv], np.float32)
    K = _store_inputs(rng, n, Hkv, D, ks, dt)
    V = _store_inputs(rng, n, Hkv, D, vs, dt)
    slots = rng.choice(S, n, replace=False).astype(np.int32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kp = torch.zeros((S, Hkv, D), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((S, Hkv, D), dtype=torch.uint8, device="cuda")
    store_kv_fp8(torch.from_numpy(K).cuda().to(tdt), torch.from_numpy(V).cuda().to(tdt),
                 torch.from_numpy(slots).cuda(), kp, vp, torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda())
    torch.cuda.synchronize()
    kg, vg = kp.cpu().numpy(), vp.cpu().numpy()
    np.testing.assert_array_equal(kg[slots], F8.quantize(K, ks))
    np.testing.assert_array_equal(vg[slots], F8.quantize(V, vs))
    untouched = np.setdiff1d(np.arange(S), slots)
    assert not kg[untouched].any() and not vg[untouched].any()
    _print(f"store fp8 {dt} Hkv={Hkv} D={D}: {n} rows bit-exact")


def _check_pools(case, res, reqs):
    """Codes of the requests' logical K/V (prefix, history and the current
    token written by the fused store) equal the oracle's codes."""
    kp, vp = case.cache.k_pool.cpu().numpy(), case.cache.v_pool.cpu().numpy()
    ks, vs = case.kv_scale
    for r in reqs:
        st = case.rows[r]
        L = int(res["L"][r])
        K, V = case.logical_kv(r, int(res["L"][r] - res["P"][r]))
        sl = st.slots[:L]
        np.testing.assert_array_equal(kp[sl], F8.quantize(K, ks))
        np.testing.assert_array_equal(vp[sl], F8.quantize(V, vs))


def _small_decode_workload(seed, Hq, Hkv, D, q_scale=1.0):
    spec = W.Spec("small_dec_fp8", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, seed, extra={"q_scale": q_scale})
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


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 128), (8, 8, 64), (16, 4, 64), (16, 4, 128),
                                     (32, 16, 128)])
def test_decode_fp8_small_flat_and_cascade(Hq, Hkv, D, q_scale=1.0):
    wl = _small_decode_workload(21, Hq, Hkv, D, q_scale)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    case.check_r2t()
    _check_pools(case, res, range(wl.B))
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode fp8 small {tag} Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 64), (16, 4, 64)])
def test_decode_fp8_cascade_stores_current_token(Hq, Hkv, D):
    # the cascade call stores the current tokens itself (in the leading
    # workgroups of its prefix-stage launch when it runs in two launches,
    # D 64 here; in a kernel of its own before the one-grid cascade)
    wl = _small_decode_workload(25, Hq, Hkv, D)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=True)
    _check_pools(case, res, range(wl.B))
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"decode fp8 cascade with store Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


def test_fork_cascade_fp8_stores_current_token():
    wl = W.fork(seed=2)
    case = GroupCase(wl, fp8=True)
    L = np.full(wl.B, 4096 + 40, np.int64)
    res = run_decode(case, L, cascade=True)
    sample = list(range(0, wl.B, 9))
    _check_pools(case, res, sample)
    reqs, O, LSE = oracle_decode(case, res, reqs=sample)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"fork fp8 cascade with store: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 64)])
def test_cascade_fp8_late_suffix_rounds(Hq, Hkv, D):
    # the workloads of test_cascade_late_suffix_rounds over an FP8 cache (one
    # grid; two launches)
    wl = late_rounds_workload(31, Hq, Hkv, D)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    case.check_r2t()
    _check_pools(case, res, range(wl.B))
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode fp8 late suffix rounds {tag} Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


def test_cascade_fp8_many_later_rounds():
    # the workload of test_cascade_many_later_rounds over an FP8 cache (D 64,
    # two launches): the suffix workgroups' later items, 64 per ballot
    wl = many_rounds_workload(39, 16, 4, 64)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=True)
    _check_pools(case, res, range(wl.B))
    reqs, O, LSE = oracle_decode(case, res)
    err = bf16_err(res["o"][reqs], O)
    lerr = float(np.max(np.abs(res["lse"][reqs] - LSE)))
    _print(f"decode fp8 many later rounds: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


def test_decode_fp8_peaky():
    # queries 8x wider: sharper softmax over the dequantised keys
    test_decode_fp8_small_flat_and_cascade(32, 8, 128, q_scale=8.0)


def _tile_edge_workload(seed, Hq, Hkv, D):
    """Prefix and context lengths on and next to the 32-key tiles and the
    1024-key splits of the FP8 kernel, group sizes leaving partial row blocks."""
    spec = W.Spec("fp8_edges", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, seed)
    members = [1, 2, 5, 9]
    prefixes = [1024, 32, 1055, 33]
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    L = np.array([1025,
                  33, 64,
                  1056, 1057, 1087, 2048, 2049,
                  34, 65, 96, 97, 1023, 1024, 1025, 2080, 4095], np.int64)
    assert len(L) == len(grp)
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, L)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64), (8, 1, 128)])
def test_decode_fp8_tile_and_split_edges(Hq, Hkv, D):
    wl = _tile_edge_workload(23, Hq, Hkv, D)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    _check_pools(case, res, range(wl.B))
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode fp8 edges {tag} Hq={Hq} Hkv={Hkv} D={D}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


def test_decode_fp8_full_size_flat_and_cascade():
    """The 256-request decode workload (16 groups of 16, prefixes 512-4096,
    contexts up to 8192, 32/8/128) over an FP8 cache: every request's output
    and log-sum-exp against the oracle over the oracle's own codes, and the
    pool codes of sampled requests bit-exact."""
    wl = W.decode(seed=0)
    case = GroupCase(wl, fp8=True)
    res = run_decode(case, wl.ctx_len.copy(), cascade=False, both=True)
    sample = sorted(set(np.random.default_rng(5).choice(wl.B, 48, replace=False).tolist() + [0, wl.B - 1]))
    _check_pools(case, res, sample)
    reqs, O, LSE = oracle_decode(case, res)
    for tag, o, l in (("flat", res["o"], res["lse"]), ("cascade", res["o_c"], res["lse_c"])):
        err = bf16_err(o[reqs], O)
        lerr = float(np.max(np.abs(l[reqs] - LSE)))
        _print(f"decode fp8 full {tag}: {len(reqs)} requests, max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("s", [1, 33, 512])
def test_fork_cascade_fp8(s):
    wl = W.fork(seed=0)
    case = GroupCase(wl, fp8=True)
    L = np.full(wl.B, 4096 + s, np.int64)
    res = run_decode(case, L, cascade=False, both=True)
    sample = list(range(0, wl.B, 5))
    reqs, O, LSE = oracle_decode(case, res, reqs=sample)
    err = bf16_err(res["o"][reqs], O)
    err_c = bf16_err(res["o_c"][reqs], O)
    _print(f"fork fp8 s={s}: flat max abs err {err:.3e}, cascade {err_c:.3e}")
    assert err <= BF16_TOL and err_c <= BF16_TOL
