"""Pins of the oracle's int8 weight-only quantiser (oracle/int8.py).

Reading (the pages name torchao's int8 weight-only mode but give no formula):
per output row s = max|w| / 127 in fp32, q = round-half-to-even(w / s)
clamped to [-127, 127], zero row -> s = 0, q = 0. Pinned against a brute-force
nearest-level search, exact ties, bounds and the model's use of s * q.
"""
import numpy as np

import synth
from oracle import OracleModel
from oracle.int8 import quantize_int8_rows
from oracle.model import bf16_to_f32

from test_oracle_model import MICRO, _rel


def _brute(w, s):
    """Nearest of the 255 levels q * s (fp64), ties to the even q; independent of rint."""
    levels = np.arange(-127, 128, dtype=np.float64)
    out = np.empty(w.shape, dtype=np.int64)
    for i, x in np.ndenumerate(w):
        d = np.abs(levels * np.float64(s) - np.float64(x))
        best = np.flatnonzero(d == d.min())
        out[i] = int(levels[best[0]]) if len(best) == 1 else int(levels[best][levels[best] % 2 == 0][0])
    return out


def test_exact_ties_round_to_even():
    # amax = 127 * 2^-7 gives s = 2^-7 exactly, so w / s is exact and (k + 1/2) s is a tie
    s = 2.0 ** -7
    ks = np.array([0, 1, 2, 3, 60, 125, -1, -2, -126], dtype=np.float64)
    w = np.concatenate([[127 * s], (ks + 0.5) * s]).astype(np.float32)[None, :]
    q, scale = quantize_int8_rows(w)
    assert scale[0] == np.float32(s)
    want = [127] + [int(k) if int(k) % 2 == 0 else int(k) + 1 for k in ks]
    assert q[0].tolist() == want


def test_matches_brute_force_nearest_level():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((6, 97)) * rng.uniform(0.01, 3.0, (6, 1))).astype(np.float32)
    q, scale = quantize_int8_rows(w)
    for r in range(w.shape[0]):
        # the fp32 quotient is what the quantiser rounds; compare on the same values
        ratio = (w[r] / scale[r]).astype(np.float32).astype(np.float64)
        assert np.array_equal(q[r].astype(np.int64), _brute(ratio, 1.0))


def test_bounds_extremes_zero_row_and_symmetry():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((8, 300)).astype(np.float32) * 0.02
    w[3] = 0.0
    q, scale = quantize_int8_rows(w)
    assert q.dtype == np.int8 and scale.dtype == np.float32
    assert scale[3] == 0 and not np.any(q[3])
    for r in range(8):
        if r == 3:
            continue
        assert np.max(np.abs(q[r])) == 127                 # the largest element lands on the last level
        assert scale[r] == np.float32(np.max(np.abs(w[r])) / np.float32(127))
        err = np.abs(w[r].astype(np.float64) - q[r].astype(np.float64) * np.float64(scale[r]))
        assert np.max(err) <= 0.5 * np.float64(scale[r]) * (1 + 1e-6)
    qn, sn = quantize_int8_rows(-w)
    assert np.array_equal(sn, scale) and np.array_equal(qn, -q)


def test_int8_model_uses_dequantised_linears():
    d = MICRO
    w = synth.gen_weights(d, 0)
    m = OracleModel(d, w, wtype="int8", dt=np.float64)
    codes, scale = m.quant["fast.0.w2"]
    assert codes.dtype == np.int8
    x = np.random.default_rng(2).standard_normal(d.ffn_dim)
    want = (codes.astype(np.float64) * scale[:, None].astype(np.float64)) @ x
    assert _rel(m.fast[0].w2(x), want) < 1e-13
    assert len(m.quant) == len(synth.linear_names(d))
    assert np.array_equal(m.w0, bf16_to_f32(w["w0"]).astype(np.float64))
