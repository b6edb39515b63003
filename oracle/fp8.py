"""float8_e4m3fn and the per-row symmetric fp8 weight quantiser (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Format (OCP 8-bit floating point, E4M3 "fn" variant, which the s2-pro-fp8 model
card names as its weight dtype in "What is this?"): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; no
infinities; S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448.

Quantiser (s2-pro-fp8 model card, "Quantization Details"): every output row of
a Linear weight gets its own fp32 scale and is stored symmetrically in e4m3fn.
The card's scale formula is lost in the page text; the reading taken is
s = max_j |w_j| / 448 in fp32, q_j = e4m3(w_j / s) with an fp32 division and
round-to-nearest-even, values beyond 448 saturate, a zero row has s = 0 and
codes 0. Dequantisation is s * dec(q).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """All 256 codes decoded to fp64 straight from the bit-field definition."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = e4m3_decode_table()
# the 127 non-negative finite values, codes 0x00..0x7E, increasing with the code
_POS = _TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp32 values (exact: every e4m3 value is an fp32 value)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> uint8 codes: nearest value, ties to the even code, saturating.

    The sign bit is the input's sign bit (so -0.0 and negatives that round to
    zero give 0x80). Input must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    neg = np.signbit(x)
    a = np.abs(x).astype(np.float64)
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # _POS[hi-1] < a <= _POS[hi]
    hi = np.clip(hi, 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)              # exact hits (covers a == 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(w: np.ndarray):
    """Per-row symmetric e4m3fn quantisation of a [rows][cols] fp32 matrix.

    Returns (codes uint8 [rows][cols], scale fp32 [rows]).
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    codes = np.zeros(w.shape, dtype=np.uint8)
    nz = scale > 0
    if np.any(nz):
        ratio = (w[nz] / scale[nz][:, None]).astype(np.float32)
        codes[nz] = e4m3_encode(ratio)
    return codes, scale
