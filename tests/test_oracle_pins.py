"""Pins of the fp64 attention oracle against things other than itself.

- closed-form hand cases (tests/golden/attention_hand_cases.json);
- a textbook special case: one request with no cached prefix and identity
  layout is dense causal attention, checked against PyTorch's
  scaled_dot_product_attention in float64 on the CPU (with the GQA head
  repeat and, for a cached prefix, an explicit bottom-right causal mask);
- invariants: the two evaluation orders agree, rows of the probability matrix
  sum to 1, merging a prefix state with a suffix state equals attention over
  the whole sequence, prefix-reused rows equal recompute-from-scratch rows.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_hand_cases():
    with open(os.path.join(GOLDEN, "attention_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        D = c["D"]
        K = np.array(c["k"], np.float32).reshape(-1, 1, D)
        V = np.array(c["v"], np.float32).reshape(-1, 1, D)
        Q = np.array(c["q"], np.float32).reshape(-1, 1, D)
        pos = np.array(c["q_pos"])
        for method in (0, 1):
            O, M, L, LSE = oracle.attention([K], [V], np.zeros(len(pos)), pos, Q, 1, 1,
                                            scale=c["scale"], method=method, threads=1)
            np.testing.assert_allclose(O[:, 0, :], np.array(c["o"]), rtol=0, atol=c["tol"],
                                       err_msg=c["name"])
            np.testing.assert_allclose(LSE[:, 0], np.array(c["lse"]), rtol=0, atol=c["tol"],
                                       err_msg=c["name"])


def _sdpa_reference(K, V, Q, pos, Hq, Hkv, scale):
    """Dense causal attention with torch SDPA in float64: keys j visible to query at t iff j <= t."""
    import torch
    L = K.shape[0]
    g = Hq // Hkv
    k = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)           # [Hkv, L, D]
    v = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)
    k = k.repeat_interleave(g, dim=0)                                        # [Hq, L, D]
    v = v.repeat_interleave(g, dim=0)
    q = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)             # [Hq, nq, D]
    mask = torch.from_numpy(np.arange(L)[None, :] <= np.asarray(pos)[:, None])   # [nq, L]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()                                        # [nq, Hq, D]


@pytest.mark.parametrize("Hq,Hkv,D,P,E", [(8, 2, 16, 0, 37), (8, 2, 16, 23, 19), (4, 4, 8, 5, 9),
                                          (8, 1, 32, 40, 24)])
def test_dense_causal_special_case_matches_sdpa(Hq, Hkv, D, P, E):
    L = P + E
    K = _rand((L, Hkv, D), 1)
    V = _rand((L, Hkv, D), 2)
    Q = _rand((E, Hq, D), 3)
    pos = np.arange(P, L)
    ref = _sdpa_reference(K, V, Q, pos, Hq, Hkv, 1.0 / np.sqrt(D))
    for method in (0, 1):
        O, _, _, _ = oracle.attention([K], [V], np.zeros(E), pos, Q, Hq, Hkv, method=method)
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_gqa_head_mapping_is_contiguous_groups():
    # With Hq=4, Hkv=2 head 1 must read KV head 0 (1 // 2), not KV head 1 (1 % 2).
    Hq, Hkv, D, L = 4, 2, 4, 6
    K = _rand((L, Hkv, D), 4)
    V = _rand((L, Hkv, D), 5)
    Q = _rand((1, Hq, D), 6)
    O, _, _, _ = oracle.attention([K], [V], [0], [L - 1], Q, Hq, Hkv)
    # single-head computation with KV head 0 for q head 1
    O1, _, _, _ = oracle.attention([K[:, 0:1]], [V[:, 0:1]], [0], [L - 1], Q[:, 1:2], 1, 1)
    np.testing.assert_allclose(O[0, 1], O1[0, 0], rtol=0, atol=1e-14)
    O3, _, _, _ = oracle.attention([K[:, 1:2]], [V[:, 1:2]], [0], [L - 1], Q[:, 3:4], 1, 1)
    np.testing.assert_allclose(O[0, 3], O3[0, 0], rtol=0, atol=1e-14)


def test_two_pass_equals_online():
    Hq, Hkv, D = 8, 2, 32
    Ks = [_rand((n, Hkv, D), 10 + n) * 3 for n in (1, 17, 130)]
    Vs = [_rand((n, Hkv, D), 20 + n) for n in (1, 17, 130)]
    row_req = [0, 1, 1, 2, 2, 2]
    row_pos = [0, 0, 16, 0, 64, 129]
    Q = _rand((6, Hq, D), 7) * 3
    a = oracle.attention(Ks, Vs, row_req, row_pos, Q, Hq, Hkv, method=0)
    b = oracle.attention(Ks, Vs, row_req, row_pos, Q, Hq, Hkv, method=1)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def test_probability_rows_sum_to_one_and_match_outputs():
    Hq, Hkv, D, L = 4, 2, 16, 50
    K = _rand((L, Hkv, D), 30) * 2
    V = _rand((L, Hkv, D), 31)
    pos = np.array([0, 1, 7, 25, 49])
    Q = _rand((len(pos), Hq, D), 32) * 2
    for h in range(Hq):
        P = oracle.attention_probs(K, pos, Q, Hq, Hkv, h)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert np.all(P[np.arange(L)[None, :] > pos[:, None]] == 0.0)
        O, _, _, _ = oracle.attention([K], [V], np.zeros(len(pos)), pos, Q, Hq, Hkv, heads=[h])
        np.testing.assert_allclose(P @ V[:, h // (Hq // Hkv), :].astype(np.float64), O[:, 0, :],
                                   rtol=0, atol=1e-13)


def test_merge_of_prefix_and_suffix_states_equals_flat():
    Hq, Hkv, D = 8, 2, 32
    L = 300
    K = _rand((L, Hkv, D), 40) * 2
    V = _rand((L, Hkv, D), 41)
    pos = np.array([100, 200, 299, 299, 299])
    split = np.array([0, 64, 150, 299, 300])       # prefix = [0, split), suffix = [split, t]
    Q = _rand((len(pos), Hq, D), 42) * 2
    req = np.zeros(len(pos))
    flat = oracle.attention([K], [V], req, pos, Q, Hq, Hkv)
    pre = oracle.attention([K], [V], req, pos, Q, Hq, Hkv, key_lo=np.zeros(len(pos)), key_hi=split)
    suf = oracle.attention([K], [V], req, pos, Q, Hq, Hkv, key_lo=split, key_hi=pos + 1)
    m, l, o = oracle.merge_states(pre[1], pre[2], pre[0], suf[1], suf[2], suf[0])
    np.testing.assert_allclose(o.reshape(flat[0].shape), flat[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose((m + np.log(l)).reshape(flat[3].shape), flat[3], rtol=1e-13, atol=1e-13)
    # merging with an empty state is the identity
    m2, l2, o2 = oracle.merge_states(flat[1], flat[2], flat[0], np.full(flat[1].shape, -np.inf),
                                     np.zeros(flat[2].shape), np.zeros(flat[0].shape))
    np.testing.assert_array_equal(o2.reshape(flat[0].shape), flat[0])


def test_prefix_reuse_equals_recompute_from_scratch():
    # extend(P, E): new rows P..P+E-1 over [prefix || new]  ==  last E rows of extend(0, P+E)
    Hq, Hkv, D, P, E = 8, 2, 16, 33, 12
    K = _rand((P + E, Hkv, D), 50)
    V = _rand((P + E, Hkv, D), 51)
    Qall = _rand((P + E, Hq, D), 52)
    full = oracle.attention([K], [V], np.zeros(P + E), np.arange(P + E), Qall, Hq, Hkv)[0]
    part = oracle.attention([K], [V], np.zeros(E), np.arange(P, P + E), Qall[P:], Hq, Hkv)[0]
    np.testing.assert_array_equal(part, full[P:])


def test_invalid_arguments_are_rejected():
    K = np.zeros((4, 2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.attention([K], [K], [0], [4], np.zeros((1, 4, 8), np.float32), 4, 2)   # t >= L
    with pytest.raises(ValueError):
        oracle.attention([K], [K], [0], [1], np.zeros((1, 3, 8), np.float32), 3, 2)   # Hq % Hkv
