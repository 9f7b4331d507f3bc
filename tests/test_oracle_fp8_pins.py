"""Pins of the oracle's FP8 (e4m3fn) KV-cache side, oracle/fp8.py, and of the
oracle's attention over a dequantised KV cache (per-head K and V factors).

Each pin is fixed by something other than the oracle itself:
  - hand-worked values of the format (tests/golden/e4m3_hand_cases.json);
  - torch's float8_e4m3fn conversions (a library routine) for decode, and
    for encode inside the clamp range;
  - brute force: the nearest of all 254 finite codes, ties to the even code;
  - round trips and the half-spacing error bound of round-to-nearest;
  - attention with power-of-two factors equals attention over the scaled
    fp32 arrays (exact), and with general factors equals torch's fp64
    scaled_dot_product_attention over the dequantised values.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as F8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_decode_hand_cases():
    for c in _golden()["decode"]:
        code = int(c["code"], 16)
        got = F8.decode(np.array([code], np.uint8))[0]
        if c["value"] == "nan":
            assert math.isnan(got), c
        else:
            want = float(c["value"])
            assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_encode_hand_cases():
    for c in _golden()["encode"]:
        y = np.array([float(c["y"])], np.float32)
        assert int(F8.encode(y)[0]) == int(c["code"], 16), c


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F8.decode(codes.numpy())
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _grid_inputs(seed):
    """Random values over the clamp range plus every midpoint of adjacent
    codes and its two float32 neighbours (the tie cases)."""
    rng = np.random.default_rng(seed)
    pos = F8.VALUES[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    parts = [rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.05,
             rng.standard_normal(20000) * 0.002, mids, -mids,
             np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))]
    return np.concatenate([np.asarray(p, np.float32) for p in parts])


def test_encode_matches_torch_cast_inside_clamp_range():
    y = _grid_inputs(1)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F8.encode(y), want)


def test_encode_is_nearest_code_ties_to_even_by_brute_force():
    rng = np.random.default_rng(2)
    pos = F8.VALUES[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2)[rng.integers(0, 126, 300)]
    y = np.concatenate([rng.uniform(-460, 460, 700), mids, -mids]).astype(np.float32)
    finite = np.array([c for c in range(256) if not np.isnan(F8.VALUES[c])])
    for v in y:
        t = min(max(float(v), -448.0), 448.0)
        d = np.abs(F8.VALUES[finite] - t)
        best = finite[d == d.min()]
        if len(best) > 1:
            # a tie between two neighbours of the same sign: the even code;
            # +0 / -0 are one value, taken with the sign of y
            mags = {int(c) & 0x7F for c in best}
            if mags == {0}:
                best = np.array([0x80 if np.signbit(v) else 0x00])
            else:
                best = np.array([c for c in best if c % 2 == 0 and (c >= 0x80) == (t < 0)])
        want = int(best[0])
        if (want & 0x7F) == 0:
            want = 0x80 if np.signbit(v) else 0x00
        assert int(F8.encode(np.array([v], np.float32))[0]) == want, (v, want)


@pytest.mark.parametrize("scale", [1.0, 0.25, 8.0, 3.0, 0.013671875 * 0.7])
def test_quantize_round_trips_every_finite_code(scale):
    finite = np.array([c for c in range(256) if not np.isnan(F8.VALUES[c])], np.uint8)
    x = (F8.VALUES[finite] * np.float32(scale)).astype(np.float32)
    got = F8.quantize(x.reshape(-1, 1, 1), np.array([scale], np.float32)).reshape(-1)
    np.testing.assert_array_equal(got, finite)


def test_quantize_uses_each_heads_own_factor():
    rng = np.random.default_rng(3)
    Hkv, D = 4, 16
    scale = np.array([0.5, 2.0, 0.0078125, 3.0], np.float32)
    codes = rng.integers(0, 256, (50, Hkv, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes
    x = (F8.decode(codes) * scale[None, :, None]).astype(np.float32)
    got = F8.quantize(x, scale)
    same = (got == codes) | (((got & 0x7F) == 0) & ((codes & 0x7F) == 0))
    assert same.all()
    # dequantize is decode * the head's factor
    np.testing.assert_array_equal(F8.dequantize(codes, scale), F8.decode(codes) * scale[None, :, None])


def test_round_to_nearest_error_bound():
    """|dequantize(quantize(x)) - x| <= half the spacing of the grid at x (plus
    the float32 rounding of x / scale), for |x / scale| <= 448."""
    rng = np.random.default_rng(4)
    scale = np.array([0.0113], np.float32)
    x = (rng.standard_normal(50000) * 1.5).astype(np.float32).reshape(-1, 1, 1)
    y = (x / scale[0]).astype(np.float32).reshape(-1)
    keep = np.abs(y) <= 448
    deq = F8.dequantize(F8.quantize(x, scale), scale).reshape(-1)[keep]
    a = np.abs(y[keep].astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_spacing = 2.0 ** (e - 3) / 2 * float(scale[0])
    err = np.abs(deq - x.reshape(-1)[keep].astype(np.float64))
    assert np.all(err <= half_spacing * (1 + 1e-6) + np.abs(x.reshape(-1)[keep]) * 2.0 ** -23)


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def test_attention_with_power_of_two_factors_equals_prescaled_arrays():
    rng = np.random.default_rng(5)
    Hq, Hkv, D, L = 8, 4, 16, 37
    Kc, Vc = _rand_codes(rng, (L, Hkv, D)), _rand_codes(rng, (L, Hkv, D))
    ks = np.array([2.0 ** -7, 2.0 ** -3, 0.5, 4.0], np.float32)
    vs = np.array([2.0, 2.0 ** -6, 1.0, 2.0 ** -9], np.float32)
    Q = rng.standard_normal((6, Hq, D)).astype(np.float32)
    pos = [0, 1, 5, 17, 35, 36]
    K = F8.decode(Kc).astype(np.float32)
    V = F8.decode(Vc).astype(np.float32)
    O1, M1, L1, S1 = oracle.attention([K], [V], [0] * 6, pos, Q, Hq, Hkv, kv_scale=(ks, vs))
    Kp = (K * ks[None, :, None]).astype(np.float32)   # exact: power-of-two factors
    Vp = (V * vs[None, :, None]).astype(np.float32)
    O2, M2, L2, S2 = oracle.attention([Kp], [Vp], [0] * 6, pos, Q, Hq, Hkv)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(S1, S2)


def test_attention_with_general_factors_matches_sdpa_fp64():
    rng = np.random.default_rng(6)
    Hq, Hkv, D, L = 8, 2, 32, 29
    Kc, Vc = _rand_codes(rng, (L, Hkv, D)), _rand_codes(rng, (L, Hkv, D))
    ks = np.array([0.0137, 0.0291], np.float32)
    vs = np.array([0.0071, 0.113], np.float32)
    Q = (rng.standard_normal((L, Hq, D)) * 0.5).astype(np.float32)
    pos = np.arange(L)
    O, _, _, _ = oracle.attention([F8.decode(Kc).astype(np.float32)], [F8.decode(Vc).astype(np.float32)],
                                  [0] * L, pos, Q, Hq, Hkv, kv_scale=(ks, vs))
    Kd = torch.from_numpy(F8.dequantize(Kc, ks))                  # [L, Hkv, D] fp64
    Vd = torch.from_numpy(F8.dequantize(Vc, vs))
    g = Hq // Hkv
    Kh = Kd.permute(1, 0, 2).repeat_interleave(g, 0)             # [Hq, L, D]
    Vh = Vd.permute(1, 0, 2).repeat_interleave(g, 0)
    Qh = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh, is_causal=True).permute(1, 0, 2)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
