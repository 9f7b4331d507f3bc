"""FP8 KV cache codes -- oracle side (plain numpy).

TEST INFRASTRUCTURE ONLY: like the rest of oracle/, only tests/,
__graft_entry__.smoke() and the cpu_baseline leg of bench.py may import this.

The pages say only that SGLang can keep the KV cache in FP8, which halves it
("SGLang 深度拆解" (chenxutan.com) section 4.3, on compressing the KV cache
before it is moved; "Lecture 16 · 案例研究：SGLang" (semidirectx.com), section 4
"More engineering", lists an FP8 KV cache among the v0.3 kernel work).  They fix
neither the 8-bit format nor the scaling.  Readings taken here:

  * Format: OCP 8-bit floating point e4m3fn -- sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits.  Exponent field 0 holds the subnormals
    m * 2^-9; exponent field e >= 1 holds (1 + m/8) * 2^(e - 7).  There is no
    infinity; S.1111.111 is NaN, so the largest finite magnitude is
    1.75 * 2^8 = 448 (code 0x7e).
  * Scaling: one float32 factor per KV head for K and one for V.  The code c
    stored for head kv stands for decode(c) * scale[kv].
  * Quantisation of an input x of head kv: y = x / scale[kv] in float32
    (IEEE division, round to nearest even); y is clamped to [-448, 448] (an
    infinity clamps too); then y is rounded to the nearest e4m3fn value, a
    tie going to the even code.  The sign of y is kept, so a negative y that
    rounds to zero gives the code of -0 (0x80).  NaN inputs are outside the
    contract (quantize() rejects them).

Everything here is by enumeration of the 256 codes from their bit fields --
no bit tricks -- so that each step can be checked against the format's
definition by eye.
"""
import numpy as np

MAX_FINITE = 448.0


def _code_value(c: int) -> float:
    """Value of one e4m3fn code, straight from its bit fields."""
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9                      # subnormal: (m / 8) * 2^(1 - 7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if sign else mag


#: value of every code 0..255 (float64; NaN at 0x7f and 0xff)
VALUES = np.array([_code_value(c) for c in range(256)], dtype=np.float64)

# the non-negative finite codes 0x00..0x7e in increasing order of value
_POS = VALUES[:0x7F]
assert np.all(np.diff(_POS) > 0)


def decode(codes) -> np.ndarray:
    """float64 values of uint8 codes (any shape)."""
    return VALUES[np.asarray(codes, dtype=np.uint8)]


def encode(y) -> np.ndarray:
    """Round float32 values y (already divided by their scale) to e4m3fn codes.

    Clamp to [-448, 448], then nearest value with ties to the even code; the
    sign of y is kept.  Returns uint8 codes of y's shape.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.isnan(y).any():
        raise ValueError("fp8.encode: NaN input")
    a = np.minimum(np.abs(y.astype(np.float64)), MAX_FINITE)
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[hi], hi, code).astype(np.uint8)   # exact values
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """Codes of KV rows x [..., Hkv, D] (float32 values) with per-head scales [Hkv].

    y = x / scale[kv] in float32, then encode(y).
    """
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32).reshape(-1)
    assert x.ndim >= 2 and x.shape[-2] == s.shape[0]
    y = np.divide(x, s[:, None], dtype=np.float32)
    return encode(y)


def dequantize(codes, scale) -> np.ndarray:
    """float64 values decode(codes[..., kv, :]) * scale[kv] (exact in fp64)."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(-1)
    return decode(codes) * s[:, None]
