"""Pins for the oracle's e4m3fn codec and per-row quantiser.

Checked against: the format's defining values (OCP E4M3: bias 7, subnormals
m * 2^-9, max 448, NaN at S.1111.111), a library routine (torch's CPU
float8_e4m3fn cast), round-trip error bounds that follow from 3 mantissa bits,
and the s2-pro-fp8 model card's "Quantization Details" (201 Linear matrices
in the slow and fast backbones; tables and norms not quantised).
"""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_decode_table, e4m3_encode, quantize_rows
from synth import DIMS, linear_names, tensor_specs


def test_decode_table_defining_values():
    t = e4m3_decode_table()
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9                 # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x38] == 1.0                       # exponent field 7 == bias
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2             # no infinities, only two NaNs
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)             # codes order the values


def test_decode_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode_table()
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(both_nan, np.isnan(ref))
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(5)
    t = e4m3_decode_table()
    pos = t[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 3,
        mids, -mids,
        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_encode_ties_go_to_even_code_and_saturate():
    assert e4m3_encode(np.float32([2.0 ** -10]))[0] == 0x00     # half the smallest subnormal
    assert e4m3_encode(np.float32([3 * 2.0 ** -10]))[0] == 0x02  # between codes 1 and 2
    assert e4m3_encode(np.float32([1.0 + 1 / 16]))[0] == 0x38    # between 1 and 1.125
    assert e4m3_encode(np.float32([1.0 + 3 / 16]))[0] == 0x3A    # between 1.125 and 1.25
    assert e4m3_encode(np.float32([464.0]))[0] == 0x7E
    assert e4m3_encode(np.float32([1e30]))[0] == 0x7E
    assert e4m3_encode(np.float32([-1e30]))[0] == 0xFE
    assert e4m3_encode(np.float32([-0.0]))[0] == 0x80


def test_quantize_rows_bounds():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[5, 17] = 0.5                                   # an outlier row
    codes, s = quantize_rows(w)
    assert s.dtype == np.float32 and s[3] == 0 and np.all(codes[3] == 0)
    nz = np.arange(64) != 3
    amax = np.abs(w[nz]).max(axis=1)
    assert np.array_equal(s[nz], (amax / np.float32(448)).astype(np.float32))
    # the largest entry of each row lands on +-448
    idx = np.abs(w[nz]).argmax(axis=1)
    top = codes[nz][np.arange(63), idx]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # round trip: half an ulp of 3 mantissa bits (relative 2^-4) for normals,
    # half the subnormal step (2^-10 * s) below 2^-6 * s, plus fp32 slack
    deq = e4m3_decode(codes) * s[:, None]
    err = np.abs(deq - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6) + 1e-12
    assert np.all(err <= bound)
    assert np.all(np.sign(deq[np.abs(deq) > 0]) == np.sign(w[np.abs(deq) > 0]))


def test_201_linear_matrices_at_full_shape():
    dual = DIMS["s2pro_dual"]
    names = linear_names(dual)
    assert len(names) == 201
    assert "fast.head" in names and "w0" not in names
    kinds = {k for n, _, k in tensor_specs(dual) if n not in names}
    assert kinds == {"emb", "norm"}


@pytest.mark.parametrize("scale", [1e-3, 0.02, 1.0])
def test_quantize_is_scale_equivariant(scale):
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 256)) * scale).astype(np.float32)
    c1, s1 = quantize_rows(w)
    c2, s2 = quantize_rows((w * np.float32(2.0 ** 4)).astype(np.float32))
    assert np.array_equal(c1, c2)                    # power-of-two rescale is exact
    assert np.allclose(s2, s1 * 16, rtol=0)
