"""Pins for the oracle's building blocks against closed forms and brute force.

RMSNorm, SiLU and RoPE are checked against identities that any correct version
satisfies and a plausible bug (wrong axis, missing eps, swapped pair, sign
error, wrong frequency exponent) breaks. Attention is checked against an
explicit fp64 loop written from the softmax definition, plus special cases with
known answers, and GQA against MHA with repeated KV heads.
"""
import math

import numpy as np
import pytest

from oracle import apply_rope, gqa_attention, greedy_argmax, Linear, rmsnorm, rope_cos_sin, silu


def test_rmsnorm_constant_vector_closed_form():
    d, c, eps = 64, 0.37, 1e-6
    g = np.linspace(0.5, 1.5, d).astype(np.float64)
    y = rmsnorm(np.full(d, c, dtype=np.float64), g, eps)
    assert np.allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 256))
    ones = np.ones(256)
    y = rmsnorm(x, ones, 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-6)
    assert np.allclose(rmsnorm(17.0 * x, ones, 1e-6), y, rtol=1e-6)
    # eps matters for tiny inputs: rms(1e-4 * e) is damped by sqrt(1e-8 + 1e-6)
    t = rmsnorm(np.full(4, 1e-4), np.ones(4), 1e-6)
    assert np.allclose(t, 1e-4 / math.sqrt(1e-8 + 1e-6))


def test_silu_closed_forms():
    a = np.linspace(-20, 20, 401)
    s = silu(a)
    assert s[200] == 0.0
    assert np.allclose(s - silu(-a), a, atol=1e-12)           # a*sig(a) - (-a)*sig(-a) = a
    assert np.allclose(s, a / (1 + np.exp(-a)), rtol=1e-15)
    assert abs(silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-15


def _rope(v, p, base):
    cos, sin = rope_cos_sin([p], v.shape[-1], base, np.float64)
    return apply_rope(v, cos[0], sin[0])


def test_rope_identity_at_zero_and_pair_norms():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(128)
    assert np.array_equal(_rope(v, 0, 1e6), v)
    r = _rope(v, 777, 1e6)
    half = 64
    n0 = v[:half] ** 2 + v[half:] ** 2
    n1 = r[:half] ** 2 + r[half:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def test_rope_head_dim_two_is_a_plane_rotation_by_position():
    # hd = 2: one pair, frequency base^0 = 1, so the angle is the position itself
    for p in (0, 1, 5, 1000):
        v = np.array([0.3, -1.2])
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(_rope(v, p, 1e6), [c * 0.3 - s * -1.2, s * 0.3 + c * -1.2], rtol=1e-12)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    for m, n in [(5, 3), (100, 37), (1023, 0), (512, 511)]:
        lhs = _rope(q, m, 1e6) @ _rope(k, n, 1e6)
        rhs = _rope(q, m - n, 1e6) @ k
        assert abs(lhs - rhs) < 1e-9


def test_rope_frequency_exponent():
    # the last pair rotates by p * base^(-2(hd/2-1)/hd); the first by p
    hd, base, p = 8, 1e6, 3.0
    cos, sin = rope_cos_sin([p], hd, base, np.float64)
    assert np.allclose(np.arctan2(sin[0, 0], cos[0, 0]), p - 2 * math.pi * round(p / (2 * math.pi)))
    want = p * base ** (-2 * 3 / hd)
    assert abs(math.atan2(sin[0, 3], cos[0, 3]) - want) < 1e-12


def _brute_attention(q, k, v, q_pos):
    """Explicit fp64 loops from the definition softmax(q.k / sqrt(hd)) v."""
    n, n_q, hd = q.shape
    T, n_kv, _ = k.shape
    g = n_q // n_kv
    out = np.zeros((n, n_q, hd))
    for i in range(n):
        for h in range(n_q):
            kv = h // g
            scores = []
            for j in range(int(q_pos[i]) + 1):
                s = 0.0
                for e in range(hd):
                    s += float(q[i, h, e]) * float(k[j, kv, e])
                scores.append(s / math.sqrt(hd))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            z = sum(w)
            for e in range(hd):
                out[i, h, e] = sum(w[j] * float(v[j, kv, e]) for j in range(len(w))) / z
    return out


@pytest.mark.parametrize("n_q,n_kv,T", [(4, 2, 7), (4, 1, 3), (2, 2, 16)])
def test_attention_matches_brute_force(n_q, n_kv, T):
    rng = np.random.default_rng(3)
    hd = 8
    k = rng.standard_normal((T, n_kv, hd))
    v = rng.standard_normal((T, n_kv, hd))
    q_pos = np.array([T - 3, T - 2, T - 1]) if T >= 3 else np.array([T - 1])
    q = rng.standard_normal((len(q_pos), n_q, hd)) * 2
    got = gqa_attention(q, k, v, q_pos)
    assert np.allclose(got, _brute_attention(q, k, v, q_pos), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    hd = 16
    # a single cached position: output is that value row, whatever the query
    k = rng.standard_normal((1, 2, hd))
    v = rng.standard_normal((1, 2, hd))
    q = rng.standard_normal((1, 4, hd)) * 10
    o = gqa_attention(q, k, v, np.array([0]))
    assert np.allclose(o[0, :2], v[0, 0]) and np.allclose(o[0, 2:], v[0, 1])
    # identical keys: uniform weights, output is the mean of the visible values
    T = 9
    k = np.repeat(rng.standard_normal((1, 1, hd)), T, axis=0)
    v = rng.standard_normal((T, 1, hd))
    o = gqa_attention(rng.standard_normal((1, 2, hd)), k, v, np.array([5]))
    assert np.allclose(o[0, 0], v[:6, 0].mean(axis=0)) and np.allclose(o[0, 1], v[:6, 0].mean(axis=0))


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(6)
    n_q, n_kv, hd, T = 8, 2, 16, 11
    k = rng.standard_normal((T, n_kv, hd))
    v = rng.standard_normal((T, n_kv, hd))
    q = rng.standard_normal((2, n_q, hd))
    pos = np.array([4, 10])
    gqa = gqa_attention(q, k, v, pos)
    mha = gqa_attention(q, np.repeat(k, n_q // n_kv, axis=1), np.repeat(v, n_q // n_kv, axis=1), pos)
    assert np.allclose(gqa, mha, rtol=1e-13)


def test_linear_against_fp64_sums_and_fp8_scale_factoring():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((6, 40))
    x = rng.standard_normal(40)
    want = np.array([sum(w[r, c] * x[c] for c in range(40)) for r in range(6)])
    assert np.allclose(Linear(w)(x), want, rtol=1e-12)
    s = rng.uniform(0.1, 2, 6)
    assert np.allclose(Linear(w, s)(x), want * s, rtol=1e-12)
    assert np.allclose(Linear(w)(np.stack([x, 2 * x])), np.stack([want, 2 * want]), rtol=1e-12)


def test_greedy_argmax_first_index_and_nan():
    assert greedy_argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert greedy_argmax(np.array([np.nan, -5.0, -7.0])) == 1
    assert greedy_argmax(np.array([-np.inf, -np.inf])) == 0


def test_round_bf16_nearest_even():
    from oracle import round_bf16
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                       # bf16 spacing at 1
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9, -1 - 2.0 ** -8, 3e38, 1e-40],
                 dtype=np.float32)
    r = round_bf16(x)
    assert r[0] == one
    assert r[1] == one                                # tie -> even (1.0)
    assert r[2] == one + 2 * ulp                      # tie -> even (1 + 2^-6)
    assert r[3] == one                                # below half
    assert r[4] == -one                               # tie -> even
    assert np.isfinite(r[5]) or r[5] == np.inf
    assert r[6] >= 0
    # every value is representable: low 16 bits clear
    assert np.all(r.view(np.uint32) & 0xFFFF == 0)
    # agrees with torch's bf16 cast (a library routine) on random values
    import torch
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(v), ref)


def test_bf16_to_f32_every_bit_pattern():
    """The widening every bf16 weight goes through, over all 65,536 patterns.

    bf16 is the upper half of an IEEE binary32 word (same sign, exponent and
    top seven fraction bits), so the widening is exact. Checked against torch's
    own uint16 -> bfloat16 view -> float32 cast (a library routine): finite
    values, infinities and zeros bit for bit, NaNs by class (NaN in, NaN out,
    sign kept), plus hand-decoded patterns from the format definition.
    """
    import torch
    from oracle import bf16_to_f32
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = bf16_to_f32(bits)
    assert got.dtype == np.float32 and got.shape == bits.shape
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))
    # exponent 0x7F, fraction 0 -> 1; 0x4049 -> 3.140625; 0xC000 -> -2;
    # smallest subnormal 0x0001 -> 2^-133; 0x7F80 -> +inf; 0x8000 -> -0
    assert got[0x3F80] == 1.0 and got[0x4049] == 3.140625 and got[0xC000] == -2.0
    assert got[0x0001] == np.float32(2.0 ** -133)
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    assert got[0x8000] == 0.0 and np.signbit(got[0x8000])
    assert np.isnan(got[0x7FC0]) and np.isnan(got[0xFFFF])
