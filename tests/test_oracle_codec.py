"""Pins for the codec oracle (RVQ decode + DAC-style convolutional decoder).

Each building block is checked against something other than itself: explicit
index loops written from the definitions (brute force on tiny inputs), closed
forms (Snake, impulse responses, all-zero weights), the identity that a
transposed convolution is a plain convolution of the zero-stuffed input with
the flipped, transposed kernel, and invariants of the whole decoder that a
wrong offset, padding or stride breaks (output length, locality within the
receptive field, shift equivariance, window = full decode in the interior).
"""
import math

import numpy as np
import pytest

import synth
from oracle import (CodecParams, codec_decode, conv1d, conv_transpose1d, receptive_halo, rvq_decode,
                    snake)


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_rvq_sum_brute_force_and_first_codebook_alone():
    r = _rng(1)
    nq, V, D, T = 4, 7, 5, 6
    tables = [r.standard_normal((V, D)) for _ in range(nq)]
    codes = r.integers(0, V, size=(T, nq))
    z = rvq_decode(codes, tables)
    for t in range(T):
        for d in range(D):
            want = 0.0
            for k in range(nq):
                want += tables[k][codes[t][k]][d]
            assert abs(z[t][d] - want) < 1e-12
    # only the first (coarsest) codebook non-zero: each frame is its row
    zeros = [tables[0]] + [np.zeros((V, D))] * (nq - 1)
    assert np.array_equal(rvq_decode(codes, zeros), tables[0][codes[:, 0]])


def test_snake_closed_forms():
    alpha = np.array([0.5, 1.0, 1.3])
    x = np.zeros((1, 3))
    assert np.array_equal(snake(x, alpha), x)
    # at alpha x = pi/2 the sine term is one: x + 1/alpha
    x = (np.pi / 2 / alpha)[None, :]
    assert np.allclose(snake(x, alpha), x + 1 / alpha, rtol=0, atol=1e-12)
    # shifting x by pi/alpha shifts the output by the same amount
    v = _rng(2).standard_normal((50, 3))
    assert np.allclose(snake(v + np.pi / alpha, alpha), snake(v, alpha) + np.pi / alpha, atol=1e-12)
    # never below the identity
    assert np.all(snake(v, alpha) >= v - 1e-15)


def _conv_loops(x, w, b, dil):
    T, Cin = x.shape
    Cout, _, K = w.shape
    half = (K - 1) // 2
    y = np.zeros((T, Cout))
    for t in range(T):
        for o in range(Cout):
            acc = b[o]
            for j in range(K):
                src = t + dil * (j - half)
                if 0 <= src < T:
                    for c in range(Cin):
                        acc += w[o][c][j] * x[src][c]
            y[t][o] = acc
    return y


@pytest.mark.parametrize("K,dil,T", [(7, 1, 9), (7, 3, 11), (7, 9, 13), (1, 1, 5), (3, 2, 4)])
def test_conv1d_brute_force(K, dil, T):
    r = _rng(K * 100 + dil)
    x = r.standard_normal((T, 3))
    w = r.standard_normal((4, 3, K))
    b = r.standard_normal(4)
    assert np.allclose(conv1d(x, w, b, dil), _conv_loops(x, w, b, dil), rtol=0, atol=1e-12)


def test_conv1d_impulse_response_is_the_reversed_dilated_kernel():
    r = _rng(3)
    K, dil, T, t0 = 7, 3, 40, 20
    w = r.standard_normal((2, 1, K))
    x = np.zeros((T, 1))
    x[t0, 0] = 1.0
    y = conv1d(x, w, np.zeros(2), dil)
    want = np.zeros((T, 2))
    for j in range(K):
        want[t0 - dil * (j - 3)] = w[:, 0, j]
    assert np.array_equal(y, want)


def _convT_loops(x, w, b, s):
    T, Cin = x.shape
    _, Cout, K = w.shape
    p = s // 2
    y = np.tile(b, (T * s, 1)).astype(np.float64)
    for i in range(T):
        for k in range(K):
            o = i * s - p + k
            if 0 <= o < T * s:
                for c in range(Cin):
                    for q in range(Cout):
                        y[o][q] += x[i][c] * w[c][q][k]
    return y


@pytest.mark.parametrize("s,T", [(2, 5), (4, 3), (8, 4)])
def test_conv_transpose_brute_force_and_zero_stuffing_identity(s, T):
    r = _rng(s)
    Cin, Cout, K = 3, 2, 2 * s
    x = r.standard_normal((T, Cin))
    w = r.standard_normal((Cin, Cout, K))
    b = r.standard_normal(Cout)
    y = conv_transpose1d(x, w, b, s)
    assert y.shape == (T * s, Cout)
    assert np.allclose(y, _convT_loops(x, w, b, s), rtol=0, atol=1e-12)
    # the same as a plain correlation over the zero-stuffed input u (x[i] at
    # i*s, zeros between), left-padded by K-1-p zeros, with the flipped and
    # transposed kernel W'[q][c][m] = w[c][q][K-1-m]
    p = s // 2
    u = np.zeros(((T - 1) * s + 1, Cin))
    u[::s] = x
    lead = K - 1 - p
    upad = np.zeros((lead + T * s + K, Cin))
    upad[lead:lead + u.shape[0]] = u
    wf = np.transpose(w[:, :, ::-1], (1, 0, 2))
    z = np.tile(b, (T * s, 1)).astype(np.float64)
    for o in range(T * s):
        for m in range(K):
            z[o] += wf[:, :, m] @ upad[o + m]
    assert np.allclose(y, z, rtol=0, atol=1e-12)


@pytest.fixture(scope="module")
def tiny():
    wl = synth.CODEC_WORKLOADS["tiny_codec"]
    d = wl.dims
    return d, CodecParams(d, synth.gen_codec_weights(d, wl.weight_seed)), synth.gen_codes(wl.frames, d, wl.code_seed)


def test_decode_length_range_and_precision_modes(tiny):
    d, P, codes = tiny
    a = codec_decode(codes, P)
    assert a.shape == (codes.shape[0] * d.hop,) and d.hop == 8
    assert np.all(np.abs(a) < 1) and a.std() > 0.05
    # the bf16-activation mode stays close to fp64 (rounding of each conv input only)
    b = codec_decode(codes, P, act="bf16")
    assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-2
    assert not np.array_equal(a, b)


def test_zero_weights_give_tanh_of_the_output_bias(tiny):
    d, P, codes = tiny
    Z = CodecParams(d, {})
    for name, v in P.p.items():
        is_w = name.endswith(".w") or name.endswith(".w1") or name.endswith(".w2")
        Z.p[name] = np.zeros_like(v) if is_w else v
    y = codec_decode(codes, Z)
    assert np.allclose(y, math.tanh(P["codec.out.b"][0]), rtol=0, atol=1e-15)


def test_receptive_field_locality_and_shift_equivariance(tiny):
    d, P, _ = tiny
    h = receptive_halo(d)
    T = 100                                   # longer than two receptive fields (h = 30 frames here)
    codes = synth.gen_codes(T, d, 11)
    base = codec_decode(codes, P)
    t0 = T // 2
    c2 = codes.copy()
    c2[t0] = (c2[t0] + 1) % d.codebook_size
    diff = np.abs(codec_decode(c2, P) - base).reshape(T, d.hop).max(axis=1)
    changed = np.nonzero(diff > 0)[0]
    assert changed.size and changed.min() >= t0 - h and changed.max() <= t0 + h
    assert diff[t0] > 1e-6 and diff[0] == 0 and diff[-1] == 0
    # one frame of codes moved later moves the audio by one hop, away from the ends
    shifted = np.concatenate([codes[:1], codes[:-1]])
    s = codec_decode(shifted, P)
    lo, hi = (h + 1) * d.hop, (T - h - 1) * d.hop
    assert hi - lo > 30 * d.hop
    assert np.allclose(s[lo + d.hop:hi], base[lo:hi - d.hop], rtol=0, atol=1e-12)


def test_window_decode_equals_full_decode_in_its_interior(tiny):
    """What the full-shape GPU test relies on: frames [a, b) of a decode only
    need codes [a - halo, b + halo); a window that far out reproduces them."""
    d, P, _ = tiny
    h = receptive_halo(d)
    T = 100
    codes = synth.gen_codes(T, d, 12)
    full = codec_decode(codes, P, act="bf16")
    for a, b in [(0, 3), (T - 3, T), (T // 2 - 1, T // 2 + 1)]:
        lo, hi = max(0, a - h), min(T, b + h)
        assert hi - lo < T
        win = codec_decode(codes[lo:hi], P, act="bf16")
        got = win[(a - lo) * d.hop:(b - lo) * d.hop]
        assert np.allclose(got, full[a * d.hop:b * d.hop], rtol=0, atol=1e-9)
