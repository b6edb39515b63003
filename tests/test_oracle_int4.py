"""Pins of the oracle's int4 weight-only quantiser (oracle/int4.py).

Reading (the pages name torchao's int4 weight-only mode but give neither
formula nor group size): groups of 128 columns per row, s = max|w| / 7 in fp32,
q = round-half-to-even(w / s) clamped to [-7, 7], zero group -> 0; two codes
per byte, the even column in the low nibble. Pinned against a brute-force
nearest-level search per group, exact ties, group independence, nibble packing
written out by hand, and the model's use of s_g * q.
"""
import numpy as np

import synth
from oracle import OracleModel
from oracle.int4 import GROUP, dequantize_int4, pack_int4, quantize_int4_groups, unpack_int4

from test_oracle_model import _rel


def test_exact_ties_and_levels():
    # a group whose max is 7 * 2^-7 has s = 2^-7 exactly, so (k + 1/2) s is a tie
    s = 2.0 ** -7
    ks = np.array([0, 1, 2, 3, 5, -1, -2, -6], dtype=np.float64)
    g = np.zeros(GROUP, dtype=np.float64)
    g[0] = 7 * s
    g[1:1 + len(ks)] = (ks + 0.5) * s
    q, scale = quantize_int4_groups(g.astype(np.float32)[None, :])
    assert scale.shape == (1, 1) and scale[0, 0] == np.float32(s)
    want = [7] + [int(k) if int(k) % 2 == 0 else int(k) + 1 for k in ks]
    assert q[0, :1 + len(ks)].tolist() == want
    assert not np.any(q[0, 1 + len(ks):])


def test_matches_brute_force_per_group_and_groups_are_independent():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((3, 4 * GROUP)) * 0.02).astype(np.float32)
    w[1, GROUP + 3] = 0.9                      # an outlier in group 1 of row 1
    w[2, 2 * GROUP:3 * GROUP] = 0.0            # a zero group
    q, scale = quantize_int4_groups(w)
    levels = np.arange(-7, 8, dtype=np.float64)
    for r in range(3):
        for g in range(4):
            sl = slice(g * GROUP, (g + 1) * GROUP)
            s = scale[r, g]
            if s == 0:
                assert not np.any(q[r, sl])
                continue
            assert s == np.float32(np.max(np.abs(w[r, sl])) / np.float32(7))
            ratio = (w[r, sl] / s).astype(np.float32).astype(np.float64)
            for x, got in zip(ratio, q[r, sl]):
                d = np.abs(levels - x)
                best = levels[d == d.min()]
                want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                assert got == want
    # the outlier only coarsens its own group: the other groups of row 1 keep their scales
    ref, ref_s = quantize_int4_groups(np.delete(w[1:2], np.s_[GROUP:2 * GROUP], axis=1))
    assert np.array_equal(ref_s[0], np.delete(scale[1], 1))
    assert scale[1, 1] > 10 * scale[1, 0]
    err = np.abs(dequantize_int4(q, scale) - w.astype(np.float64))
    bound = np.repeat(scale.astype(np.float64), GROUP, axis=1) * 0.5 * (1 + 1e-6)
    assert np.all(err <= bound)


def test_nibble_packing():
    codes = np.array([[1, -1, 7, -7, 0, 3, -8 + 1, 2]], dtype=np.int8)
    packed = pack_int4(codes)
    # byte j = low nibble: column 2j, high nibble: column 2j+1 (two's complement)
    assert packed.tolist() == [[0xF1, 0x97, 0x30, 0x29]]
    assert np.array_equal(unpack_int4(packed), codes)
    rng = np.random.default_rng(6)
    c = rng.integers(-7, 8, (5, 256)).astype(np.int8)
    assert np.array_equal(unpack_int4(pack_int4(c)), c)


def test_int4_model_uses_dequantised_linears():
    d = synth.DIMS["tiny"]       # every width a multiple of the 128-column group
    w = synth.gen_weights(d, 0)
    m = OracleModel(d, w, wtype="int4", dt=np.float64)
    codes, scale = m.quant["slow.0.wqkv"]
    assert codes.shape[1] // GROUP == scale.shape[1]
    x = np.random.default_rng(7).standard_normal(d.d_model)
    want = dequantize_int4(codes, scale) @ x
    assert _rel(m.slow[0].wqkv(x), want) < 1e-13
    assert len(m.quant) == len(synth.linear_names(d))
