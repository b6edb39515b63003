"""RVQ codec decode on the GPU against the codec oracle, through the C ABI.

Single convolutions (dar_codec_op_conv: plain 7-tap at dilations 1, 3, 9, the
1-tap, transposed at strides 2, 4, 8, the one-channel output convolution; ragged
row counts and column widths that do not fill a tile) against oracle/codec.py's
conv1d / conv_transpose1d on the same bf16-rounded inputs. Whole decodes: the
tiny codec in full, and the full-shape codec (167 frames, the tuna-fish
README's 7.73 s clip padded to whole hops) on windows at the start, middle and
end, each checked against the oracle run on the window's codes plus its
receptive field (which gives the same samples; pinned on the CPU).

Tolerances. Each convolution's inputs are bf16 on both sides; the GPU sums in
fp32 on MFMA, so a convolution output may differ by fp32 summation error
(2e-5 of the sum of |w x|) plus, where the input went through Snake, the odd
input rounded to the neighbouring bf16 value because fp32 sinf and fp64 sin
straddle a rounding boundary (2^-7 of the largest |w x| term). A whole decode
chains about thirty such roundings, and a rounding decision flips wherever
fp32 and fp64 sums straddle a bf16 boundary; the flips then propagate. The
oracle itself shows the size of that: perturbing each of its convolution sums
by a relative 1e-7 (fp32 noise) moves its bf16-activation output by 0.6e-3 to
2.8e-3 relative L2 at the tiny shape and by 7.3e-3 to 7.7e-3 at full shape (a
24-frame window). So a whole decode is held to <= 1.5e-2 (about twice that
spread) against the oracle in the same activation precision and <= 2e-2
against the fp64 oracle (bf16 activation rounding alone moves the oracle's
output by 0.4% at the tiny shape and 0.8% at full shape), and each
convolution to the tight per-output bound above.
"""
import ctypes

import numpy as np
import pytest

import synth
from oracle import CodecParams, bf16_to_f32, codec_decode, conv1d, conv_transpose1d, receptive_halo, round_bf16, snake

pytestmark = pytest.mark.gpu


def _bf16_bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _dev(arr, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(dtype)).to("cuda")


def _op(x, x_bf16, alpha, w, b, taps, dil, stride, Cout, res=None, tanh=False):
    import torch
    from dar_decode_frame_amd import native as N
    T, Cin = x.shape
    xd = _dev(_bf16_bits(x), np.int16) if x_bf16 else _dev(np.asarray(x, np.float32), np.float32)
    ad = _dev(_bf16_bits(alpha), np.int16) if alpha is not None else None
    wd, bd = _dev(_bf16_bits(w), np.int16), _dev(_bf16_bits(b), np.int16)
    rows = T * stride if stride else T
    y = torch.zeros(rows, Cout, dtype=torch.float32, device="cuda")
    rd = None
    if res is not None:
        rd = _dev(np.asarray(res, np.float32), np.float32)
    torch.cuda.synchronize()
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    N.dar_codec_op_conv(p(xd), int(x_bf16), p(ad), T, Cin, Cout, p(wd), p(bd), taps, dil, stride, p(rd), int(tanh),
                        p(y), None)
    return y.cpu().numpy().astype(np.float64)


def _wide(a):
    return bf16_to_f32(_bf16_bits(a)).astype(np.float64)


@pytest.mark.parametrize("T,Cin,Cout,K,dil,snk", [
    (45, 64, 64, 7, 1, True), (150, 32, 96, 7, 9, True), (333, 96, 96, 7, 3, True), (37, 64, 128, 7, 1, False),
    (70, 64, 32, 1, 1, False), (1, 32, 64, 7, 1, True), (2000, 96, 96, 7, 9, True), (167, 1024, 1536, 7, 1, False),
    (150, 64, 96, 3, 9, True), (77, 96, 64, 5, 3, True), (300, 256, 256, 5, 2, False),
])
def test_conv_against_oracle(T, Cin, Cout, K, dil, snk):
    r = np.random.default_rng(T * 7 + Cin)
    x = r.standard_normal((T, Cin)).astype(np.float32)
    alpha = _wide(0.5 + r.random(Cin)) if snk else None
    w = _wide(r.standard_normal((Cout, Cin, K)) / np.sqrt(Cin * K))
    b = _wide(r.standard_normal(Cout) * 0.1)
    got = _op(x if snk else _wide(x), not snk, alpha, w, b, K, dil, 0, Cout)
    xin = snake(x.astype(np.float64), alpha) if snk else _wide(x)
    xin = round_bf16(xin).astype(np.float64)
    ref = conv1d(xin, w, b, dil)
    err = np.abs(got - ref)
    S = conv1d(np.abs(xin), np.abs(w), np.zeros(Cout), dil)
    assert np.all(err <= 2e-5 * S + 2.0 ** -7 * np.abs(w).max() * np.abs(xin).max()), err.max()
    if not snk:
        assert np.all(err <= 2e-5 * S + 1e-30)


@pytest.mark.parametrize("T,Cin,Cout,s", [(19, 64, 32, 2), (11, 64, 64, 4), (9, 32, 64, 8), (167, 1536, 768, 8),
                                          (1000, 192, 96, 4)])
def test_transposed_conv_against_oracle(T, Cin, Cout, s):
    r = np.random.default_rng(T + s)
    x = r.standard_normal((T, Cin)).astype(np.float32)
    alpha = _wide(0.5 + r.random(Cin))
    w = _wide(r.standard_normal((Cin, Cout, 2 * s)) / np.sqrt(2 * Cin))
    b = _wide(r.standard_normal(Cout) * 0.1)
    got = _op(x, False, alpha, w, b, 2, 1, s, Cout)
    xin = round_bf16(snake(x.astype(np.float64), alpha)).astype(np.float64)
    ref = conv_transpose1d(xin, w, b, s)
    S = conv_transpose1d(np.abs(xin), np.abs(w), np.zeros(Cout), s)
    err = np.abs(got - ref)
    assert got.shape == (T * s, Cout)
    assert np.all(err <= 2e-5 * S + 2.0 ** -7 * np.abs(w).max() * np.abs(xin).max()), err.max()


def test_residual_add_in_place_and_output_conv():
    import torch
    from dar_decode_frame_amd import native as N
    r = np.random.default_rng(5)
    T, C = 300, 64
    # residual 1-tap conv with the output aliasing the residual (in place)
    h = _wide(r.standard_normal((T, C)))
    x = r.standard_normal((T, C)).astype(np.float32)
    w = _wide(r.standard_normal((C, C, 1)) * 0.1)
    b = _wide(r.standard_normal(C) * 0.1)
    hd = _dev(_bf16_bits(h), np.int16)
    xd = _dev(x, np.float32)
    wd, bd = _dev(_bf16_bits(w), np.int16), _dev(_bf16_bits(b), np.int16)
    torch.cuda.synchronize()
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    N.dar_codec_op_conv(p(hd), 1, None, T, C, C, p(wd), p(bd), 1, 1, 0, p(xd), 0, p(xd), None)
    got = xd.cpu().numpy().astype(np.float64)
    ref = x + conv1d(h, w, b)
    S = conv1d(np.abs(h), np.abs(w), np.zeros(C)) + np.abs(x)
    assert np.all(np.abs(got - ref) <= 2e-5 * S)
    # output convolution: Snake, 7 taps to one channel, tanh; ragged sample count
    T2 = 1000
    x2 = r.standard_normal((T2, 96)).astype(np.float32)
    a2 = _wide(0.5 + r.random(96))
    w2 = _wide(r.standard_normal((1, 96, 7)) * 0.05)
    b2 = _wide(r.standard_normal(1) * 0.1)
    got2 = _op(x2, False, a2, w2, b2, 7, 1, 0, 1, tanh=True)[:, 0]
    xin = round_bf16(snake(x2.astype(np.float64), a2)).astype(np.float64)
    ref2 = np.tanh(conv1d(xin, w2, b2)[:, 0])
    assert np.max(np.abs(got2 - ref2)) < 1e-5 + 2.0 ** -7 * np.abs(w2).max() * np.abs(xin).max()


@pytest.mark.parametrize("T,C,K,x_bf16", [
    (1, 96, 7, True), (250, 96, 7, True), (251, 96, 7, False), (1000, 32, 7, True), (777, 64, 5, False),
    (513, 96, 3, True), (300, 96, 1, True), (4001, 96, 7, True), (2500, 192, 7, False), (256, 128, 7, True),
])
def test_output_conv_against_oracle(T, C, K, x_bf16):
    """The one-channel output convolution (per-row tap projections on MFMA,
    then the shifted sum over taps): both operand forms, row counts around a
    workgroup's 256 - (K - 1) outputs and ragged tails, every odd kernel size,
    widths of one to two passes over the channels. Against the oracle's conv1d
    on the same bf16 operand: fp32 summation error, plus one bf16 step of a
    Snake'd input where fp32 and fp64 Snake round differently (fp32 input)."""
    r = np.random.default_rng(T * 3 + C + K)
    x = r.standard_normal((T, C)).astype(np.float32)
    alpha = None if x_bf16 else _wide(0.5 + r.random(C))
    w = _wide(r.standard_normal((1, C, K)) * 0.05)
    b = _wide(r.standard_normal(1) * 0.1)
    got = _op(_wide(x) if x_bf16 else x, x_bf16, alpha, w, b, K, 1, 0, 1, tanh=True)[:, 0]
    xin = _wide(x) if x_bf16 else round_bf16(snake(x.astype(np.float64), alpha)).astype(np.float64)
    pre = conv1d(xin, w, b)[:, 0]
    S = conv1d(np.abs(xin), np.abs(w), np.zeros(1))[:, 0]
    bound = 2e-5 * S + 1e-7 + (0 if x_bf16 else 2.0 ** -7 * np.abs(w).max() * np.abs(xin).max())
    assert got.shape == (T,)
    assert np.all(np.abs(got - np.tanh(pre)) <= bound), np.abs(got - np.tanh(pre)).max()


@pytest.mark.parametrize("T,C,dil,taps", [(150, 32, 9, 7), (70, 64, 3, 7), (333, 96, 1, 7), (45, 128, 3, 7),
                                          (700, 96, 9, 7), (1, 96, 1, 7), (129, 128, 1, 7), (200, 96, 3, 3),
                                          (97, 64, 9, 5), (130, 128, 2, 5), (50, 32, 1, 1)])
def test_fused_residual_unit(T, C, dil, taps):
    """dar_codec_op_resunit: the one-launch unit (hidden rows kept in LDS)
    gives the two-launch path's values bit for bit, and both are within the
    oracle's bound: the dilated convolution's per-output bound e1, carried
    through Snake (slope at most 2) and the hidden bf16 rounding (a value may
    land one bf16 step, at most 2^-7 of its size, away), then summed by the
    1-tap convolution, plus fp32 summation error."""
    import torch
    from dar_decode_frame_amd import native as N
    r = np.random.default_rng(C * 1000 + T)
    x = r.standard_normal((T, C)).astype(np.float32)
    a1, a2 = _wide(0.5 + r.random(C)), _wide(0.5 + r.random(C))
    w1 = _wide(r.standard_normal((C, C, taps)) / np.sqrt(taps * C))
    b1 = _wide(r.standard_normal(C) * 0.1)
    w2 = _wide(r.standard_normal((C, C, 1)) / np.sqrt(C))
    b2 = _wide(r.standard_normal(C) * 0.1)
    xd = _dev(x, np.float32)
    dev = {k: _dev(_bf16_bits(v), np.int16) for k, v in dict(a1=a1, a2=a2, w1=w1, b1=b1, w2=w2, b2=b2).items()}
    out = {}
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    for fused in (1, 0):
        y = torch.full((T, C), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        N.dar_codec_op_resunit(p(xd), T, C, p(dev["a1"]), p(dev["w1"]), p(dev["b1"]), taps, dil, p(dev["a2"]),
                               p(dev["w2"]), p(dev["b2"]), fused, p(y), None)
        out[fused] = y.cpu().numpy()
    assert np.array_equal(out[1].view(np.uint32), out[0].view(np.uint32))
    xin = round_bf16(snake(x.astype(np.float64), a1)).astype(np.float64)
    pre = conv1d(xin, w1, b1, dil)
    e1 = 2e-5 * conv1d(np.abs(xin), np.abs(w1), np.zeros(C), dil) + 2.0 ** -7 * np.abs(w1).max() * np.abs(xin).max()
    h = round_bf16(snake(pre, a2)).astype(np.float64)
    ref = x + conv1d(h, w2, b2)
    dh = 2.0 ** -7 * np.abs(h) + 2 * e1
    bound = conv1d(dh, np.abs(w2), np.zeros(C)) + 2e-5 * (conv1d(np.abs(h), np.abs(w2), np.zeros(C)) + np.abs(x))
    err = np.abs(out[1] - ref)
    assert np.all(err <= bound), float((err / bound).max())
    # in place is refused for the one-launch kernel, allowed for two launches
    with pytest.raises(RuntimeError):
        N.dar_codec_op_resunit(p(xd), T, C, p(dev["a1"]), p(dev["w1"]), p(dev["b1"]), taps, dil, p(dev["a2"]),
                               p(dev["w2"]), p(dev["b2"]), 1, p(xd), None)
    N.dar_codec_op_resunit(p(xd), T, C, p(dev["a1"]), p(dev["w1"]), p(dev["b1"]), taps, dil, p(dev["a2"]),
                           p(dev["w2"]), p(dev["b2"]), 0, p(xd), None)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), out[0].view(np.uint32))


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.fixture(scope="module")
def tiny_codec():
    from dar_decode_frame_amd.session import CodecSession
    wl = synth.CODEC_WORKLOADS["tiny_codec"]
    d = wl.dims
    host = synth.gen_codec_weights(d, wl.weight_seed)
    sess = CodecSession(d, host, 128)
    yield d, host, CodecParams(d, host), sess
    sess.close()


@pytest.mark.parametrize("frames", [37, 1, 2, 128])
def test_tiny_decode_against_oracle(tiny_codec, frames):
    d, host, P, sess = tiny_codec
    codes = synth.gen_codes(frames, d, 3 + frames)
    got = sess.decode(codes).astype(np.float64)
    ref_b = codec_decode(codes, P, act="bf16")
    ref_f = codec_decode(codes, P)
    assert got.shape == ref_b.shape == (frames * d.hop,)
    assert np.all(np.abs(got) < 1)
    assert _rel(got, ref_b) <= 1.5e-2, _rel(got, ref_b)
    assert _rel(got, ref_f) <= 2e-2, _rel(got, ref_f)
    print(f"tiny codec {frames} frames: rel L2 {_rel(got, ref_b):.2e} (bf16 activations), {_rel(got, ref_f):.2e} (fp64)")


@pytest.mark.parametrize("frames", [23, 1])
def test_small_k5_decode_against_oracle(frames):
    """A second shape (5-tap convolutions, two residual units per block, three
    blocks, a 256-channel block on the two-launch path) against the oracle, to
    the tiny codec's bar."""
    from dar_decode_frame_amd.session import CodecSession
    d = synth.CODEC_DIMS["small_codec_k5"]
    host = synth.gen_codec_weights(d, 5)
    P = CodecParams(d, host)
    sess = CodecSession(d, host, 32)
    try:
        codes = synth.gen_codes(frames, d, 11 + frames)
        got = sess.decode(codes).astype(np.float64)
    finally:
        sess.close()
    ref_b = codec_decode(codes, P, act="bf16")
    ref_f = codec_decode(codes, P)
    assert got.shape == ref_b.shape == (frames * d.hop,)
    assert np.all(np.abs(got) < 1)
    assert _rel(got, ref_b) <= 1.5e-2, _rel(got, ref_b)
    assert _rel(got, ref_f) <= 2e-2, _rel(got, ref_f)
    print(f"small k5 codec {frames} frames: rel L2 {_rel(got, ref_b):.2e} (bf16 activations), {_rel(got, ref_f):.2e} (fp64)")


def test_tiny_decode_repeats_and_clamps_out_of_range_codes(tiny_codec):
    d, host, P, sess = tiny_codec
    codes = synth.gen_codes(40, d, 99)
    a = sess.decode(codes)
    assert np.array_equal(a, sess.decode(codes))
    before = sess.anomalies()
    bad = codes.copy()
    bad[3, 2] = d.codebook_size + 5
    bad[17, 9] = -4
    got = sess.decode(bad)
    assert sess.anomalies() - before == 2
    clamped = bad.copy()
    clamped[3, 2] = d.codebook_size - 1
    clamped[17, 9] = 0
    assert np.array_equal(got, sess.decode(clamped))


def test_capacity_and_argument_errors(tiny_codec):
    import torch
    from dar_decode_frame_amd import native as N
    d, host, P, sess = tiny_codec
    codes = torch.zeros(200, d.n_codebooks, dtype=torch.int32, device="cuda")
    audio = torch.zeros(200 * d.hop, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    with pytest.raises(N.DarError) as e:
        N.dar_codec_decode(sess.ctx, p(codes), 129, p(audio))
    assert e.value.status == N.DAR_E_CAPACITY
    with pytest.raises(N.DarError) as e:
        N.dar_codec_decode(sess.ctx, p(codes), 0, p(audio))
    assert e.value.status == N.DAR_E_INVAL


def test_fullshape_decode_windows_against_oracle():
    """The 7.73 s clip (167 frames) at full shape: three windows of four frames
    (start, middle, end), each against the oracle over the window plus its
    receptive field."""
    from dar_decode_frame_amd.session import CodecSession
    wl = synth.CODEC_WORKLOADS["s2pro_codec_7s"]
    d = wl.dims
    host = synth.gen_codec_weights(d, wl.weight_seed)
    codes = synth.gen_codes(wl.frames, d, wl.code_seed)
    sess = CodecSession(d, host, wl.frames)
    got = sess.decode(codes).astype(np.float64)
    sess.close()
    assert got.shape == (wl.frames * d.hop,) and np.all(np.abs(got) < 1)
    P = CodecParams(d, host)
    h = receptive_halo(d)
    T = wl.frames
    for a, b in [(0, 4), (T // 2 - 2, T // 2 + 2), (T - 4, T)]:
        lo, hi = max(0, a - h), min(T, b + h)
        seg = slice(a * d.hop, b * d.hop)
        win = slice((a - lo) * d.hop, (b - lo) * d.hop)
        ref_b = codec_decode(codes[lo:hi], P, act="bf16")[win]
        ref_f = codec_decode(codes[lo:hi], P)[win]
        rb, rf = _rel(got[seg], ref_b), _rel(got[seg], ref_f)
        print(f"full-shape codec frames {a}..{b}: rel L2 {rb:.2e} (bf16 activations), {rf:.2e} (fp64)")
        assert rb <= 1.5e-2 and rf <= 2e-2
