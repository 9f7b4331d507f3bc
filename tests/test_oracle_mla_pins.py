"""Pins of the oracle's attention in a latent space (value width Dv different
from the score width D), the form the pages give for DeepSeek's MLA: the
decompression matrices are absorbed into the query and output projections and
attention runs directly on the 576-dim latent ("Lecture 16 · 案例研究：SGLang"
(semidirectx.com) section 4, "More engineering").  Each pin is fixed by
something other than the oracle:
  - a closed form with D = 2, Dv = 1;
  - torch's fp64 scaled_dot_product_attention (a library routine, value width
    free) on the 576/512 shape;
  - the absorption identity itself: per-head attention over decompressed keys
    and values equals latent attention with absorbed queries, projected back.
"""
import math

import numpy as np
import torch

import oracle


def test_closed_form_value_width_one():
    # keys (0, 0) and (ln 3, 5); values 2 and 10 (first value dim of the latent
    # [v, extra]); q = (1, 0), scale 1: weights 1/4, 3/4 -> o = 0.5 + 7.5 = 8;
    # lse = ln(1 + 3) = ln 4
    K = np.array([[[0.0, 0.0]], [[math.log(3.0), 5.0]]], np.float32)
    V = np.array([[[2.0]], [[10.0]]], np.float32)
    O, M, Ls, LSE = oracle.attention([K], [V], [0], [1], np.array([[[1.0, 0.0]]], np.float32), 1, 1, scale=1.0)
    assert O.shape == (1, 1, 1)
    assert abs(O[0, 0, 0] - 8.0) < 1e-6 and abs(LSE[0, 0] - math.log(4.0)) < 1e-6


def test_latent_576_512_matches_sdpa_fp64():
    rng = np.random.default_rng(1)
    Hq, L, D, Dv = 16, 57, 576, 512
    lat = (rng.standard_normal((L, 1, D)) * 0.5).astype(np.float32)
    Q = (rng.standard_normal((4, Hq, D)) * 0.5).astype(np.float32)
    pos = [0, 9, 33, 56]
    scale = 1.0 / math.sqrt(192.0)
    O, _, _, LSE = oracle.attention([lat], [np.ascontiguousarray(lat[:, :, :Dv])], [0] * 4, pos, Q, Hq, 1,
                                    scale=scale)
    for i, t in enumerate(pos):
        k = torch.from_numpy(lat[:t + 1, 0].astype(np.float64))             # [t+1, D]
        v = k[:, :Dv]
        q = torch.from_numpy(Q[i].astype(np.float64))                       # [Hq, D]
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], scale=scale)[0]
        np.testing.assert_allclose(O[i], ref.numpy(), rtol=0, atol=1e-12)
        s = (q @ k.T) * scale
        np.testing.assert_allclose(LSE[i], torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_weight_absorption_identity():
    # per head h: key k_jh = [W_uk[h] c_j || r_j], value v_jh = W_uv[h] c_j,
    # query q_h = [qn_h || qr_h].  Absorbed: q'_h = [W_uk[h]^T qn_h || qr_h]
    # over the latent [c_j || r_j] gives the same scores, and W_uv[h] applied to
    # the latent output gives the same values.
    rng = np.random.default_rng(2)
    Hq, L, dc, dr, dn, dv = 4, 23, 12, 4, 6, 5
    c = rng.standard_normal((L, dc))
    r = rng.standard_normal((L, dr))
    W_uk = rng.standard_normal((Hq, dn, dc)) * 0.3
    W_uv = rng.standard_normal((Hq, dv, dc)) * 0.3
    qn = rng.standard_normal((Hq, dn))
    qr = rng.standard_normal((Hq, dr))
    t, scale = L - 1, 1.0 / math.sqrt(dn + dr)
    # per-head form (Hkv = Hq, one KV head per query head)
    K = np.stack([np.concatenate([c @ W_uk[h].T, r], 1) for h in range(Hq)], 1).astype(np.float32)
    V = np.stack([c @ W_uv[h].T for h in range(Hq)], 1).astype(np.float32)
    Qh = np.concatenate([qn, qr], 1)[None].astype(np.float32)
    O1, _, _, L1 = oracle.attention([K], [V], [0], [t], Qh, Hq, Hq, scale=scale)
    # latent form: one KV head [c || r], values = c, absorbed queries
    lat = np.concatenate([c, r], 1)[:, None, :].astype(np.float32)
    Qa = np.stack([np.concatenate([W_uk[h].T @ qn[h], qr[h]]) for h in range(Hq)])[None].astype(np.float32)
    O2, _, _, L2 = oracle.attention([lat], [np.ascontiguousarray(lat[:, :, :dc])], [0], [t], Qa, Hq, 1,
                                    scale=scale)
    O2p = np.stack([W_uv[h] @ O2[0, h] for h in range(Hq)])[None]
    # the two forms round the float32 inputs differently (K vs its factors), so
    # they agree to float32 input precision, not exactly
    np.testing.assert_allclose(O2p, O1, rtol=0, atol=2e-5)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=2e-5)
