"""Per-kernel parity of the HIP library against the oracle, through the C ABI.

Bars: fp8 decode and the fp8, int8 and int4 quantisers are integer/byte work, so bit-exact;
GEMV and attention are fp32 accumulations checked against the oracle in fp64
on the same bf16 / fp8 inputs, within a bound derived from fp32 summation
(|error| <= 1e-5 * sum_j |w_j x_j|, and 2e-5 relative for attention).
"""
import ctypes

import numpy as np
import pytest

import synth
from oracle import e4m3_decode, e4m3_decode_table, gqa_attention, quantize_rows
from oracle.int4 import dequantize_int4, pack_int4, quantize_int4_groups
from oracle.int8 import quantize_int8_rows
from oracle.model import bf16_to_f32

WT_CODES = {"bf16": 0, "fp8": 1, "int8": 2, "int4": 3}
QTYPES = ["bf16", "fp8", "int8", "int4"]


def _quantised(wtype, w32):
    """(device codes array, fp32 scales, fp64 weights before the row scale, fp64
    row scale) of the oracle's quantiser; int4's group scales are inside the weights."""
    if wtype == "fp8":
        codes, scale = quantize_rows(w32)
        return codes, scale, e4m3_decode(codes).astype(np.float64), scale.astype(np.float64)
    if wtype == "int4":
        codes, scale = quantize_int4_groups(w32)
        return pack_int4(codes), scale, dequantize_int4(codes, scale), np.ones(w32.shape[0])
    codes, scale = quantize_int8_rows(w32)
    return codes, scale, codes.astype(np.float64), scale.astype(np.float64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from dar_decode_frame_amd import native as N
    dev = torch.device("cuda:0")
    return torch, N, dev


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _sp(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bf16_matrix(rows, cols, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_normal((rows, cols)) * scale).astype(np.float32))


def test_stream_read_reference(env):
    """dar_op_stream_read: a plain read of 64 MiB (the fastest of its launch
    shapes) reports a rate a read can have (between 0.2 and 10 TB/s on this
    part), leaves the sink alone (its marker value needs a read that sums to
    it), handles a buffer smaller than a grid stride, and rejects bad
    arguments."""
    torch, N, dev = env
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    sink = torch.full((2048,), 7, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    N.dar_op_stream_read(_p(buf), buf.numel(), 1, _p(sink), _sp(torch))  # the first launch loads the kernel
    ms = N.dar_op_stream_read(_p(buf), buf.numel(), 3, _p(sink), _sp(torch))
    rate = buf.numel() / (ms * 1e-3)
    assert 0.2e12 < rate < 10e12, rate
    assert bool((sink == 7).all())
    # smaller than one grid stride of every shape: only the loops' tails read
    ms_small = N.dar_op_stream_read(_p(buf), 4096, 2, _p(sink), _sp(torch))
    assert ms_small > 0 and bool((sink == 7).all())
    out = ctypes.c_float(0)
    assert N.lib.dar_op_stream_read(_p(buf), 100, 1, _p(sink), ctypes.byref(out), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(_p(buf), 1024, 0, _p(sink), ctypes.byref(out), None) == N.DAR_E_INVAL


def test_fp8_decode_all_codes(env):
    torch, N, dev = env
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(dev)
    out = torch.empty(256, dtype=torch.float32, device=dev)
    N.dar_op_fp8_decode(_p(codes), 256, _p(out), _sp(torch))
    got = out.cpu().numpy().astype(np.float64)
    want = e4m3_decode_table()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), np.nonzero(np.isnan(got) != nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("rows,cols", [(7, 256), (96, 2560), (33, 9728)])
def test_quantizer_bit_exact(env, rows, cols):
    torch, N, dev = env
    bits = _bf16_matrix(rows, cols, 100 + rows)
    bits[1] = 0                                   # zero row
    bits[2, 5] = 0x8000                           # negative zero
    bits[3, 9] = synth.f32_to_bf16_bits(np.float32([0.9]))[0]   # outlier
    w = torch.from_numpy(bits.view(np.int16)).to(dev)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s = torch.empty(rows, dtype=torch.float32, device=dev)
    N.dar_quantize_fp8_rows(_p(w), rows, cols, _p(q), _p(s), _sp(torch))
    torch.cuda.synchronize()
    codes, scale = quantize_rows(bf16_to_f32(bits))
    assert np.array_equal(s.cpu().numpy(), scale)
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("rows,cols", [(7, 256), (96, 2560), (33, 9728)])
def test_int8_quantizer_bit_exact(env, rows, cols):
    torch, N, dev = env
    bits = _bf16_matrix(rows, cols, 200 + rows)
    bits[1] = 0                                   # zero row
    bits[2, 5] = 0x8000                           # negative zero
    bits[3, 9] = synth.f32_to_bf16_bits(np.float32([0.9]))[0]   # outlier
    w = torch.from_numpy(bits.view(np.int16)).to(dev)
    q = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    s = torch.empty(rows, dtype=torch.float32, device=dev)
    N.dar_quantize_int8_rows(_p(w), rows, cols, _p(q), _p(s), _sp(torch))
    torch.cuda.synchronize()
    codes, scale = quantize_int8_rows(bf16_to_f32(bits))
    assert np.array_equal(s.cpu().numpy(), scale)
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("rows,cols", [(7, 256), (96, 2560), (33, 9728)])
def test_int4_quantizer_bit_exact(env, rows, cols):
    torch, N, dev = env
    bits = _bf16_matrix(rows, cols, 300 + rows)
    bits[1] = 0                                   # zero row
    bits[2, 128:256] = 0                          # one zero group
    bits[2, 5] = 0x8000                           # negative zero
    bits[3, 9] = synth.f32_to_bf16_bits(np.float32([0.9]))[0]   # outlier
    w = torch.from_numpy(bits.view(np.int16)).to(dev)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device=dev)
    N.dar_quantize_int4_groups(_p(w), rows, cols, _p(q), _p(s), _sp(torch))
    torch.cuda.synchronize()
    codes, scale = quantize_int4_groups(bf16_to_f32(bits))
    assert np.array_equal(s.cpu().numpy(), scale)
    assert np.array_equal(q.cpu().numpy(), pack_int4(codes))


GEMV_SHAPES = [(512, 256), (300, 768), (6144, 2560), (2560, 4096), (9728, 2560), (2560, 9728), (4096, 2560),
               (33, 3072), (17, 13312)]  # last two: ragged rows over chunk counts split unevenly across waves


@pytest.mark.parametrize("wtype", QTYPES)
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("rows,cols", GEMV_SHAPES)
def test_gemv_against_fp64(env, wtype, M, rows, cols):
    torch, N, dev = env
    bits = _bf16_matrix(rows, cols, rows * 7 + cols)
    w32 = bf16_to_f32(bits)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((M, cols)).astype(np.float32)
    xt = torch.from_numpy(x).to(dev)
    y = torch.full((M, rows), float("nan"), dtype=torch.float32, device=dev)
    if wtype == "bf16":
        w_dev = torch.from_numpy(bits.view(np.int16)).to(dev)
        N.dar_op_gemv(0, _p(w_dev), None, rows, cols, _p(xt), M, _p(y), _sp(torch))
        w_ref = w32.astype(np.float64)
        sc = np.ones(rows)
    else:
        codes, scale, w_ref, sc = _quantised(wtype, w32)
        w_dev = torch.from_numpy(codes).to(dev)
        s_dev = torch.from_numpy(scale).to(dev)
        N.dar_op_gemv(WT_CODES[wtype], _p(w_dev), _p(s_dev), rows, cols, _p(xt), M, _p(y), _sp(torch))
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    want = (x.astype(np.float64) @ w_ref.T) * sc
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(w_ref).T) * sc + 1e-30
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) / bound))


# prefill GEMM: full blocks, ragged rows (M not a multiple of 32), narrow and
# wide outputs (K split across workgroups), the frame's shapes
GEMM_SHAPES = [(6144, 2560, 128), (2560, 4096, 128), (9728, 2560, 100), (2560, 9728, 7), (300, 768, 33),
               (17, 256, 1), (129, 512, 64)]


@pytest.mark.parametrize("wtype", QTYPES)
@pytest.mark.parametrize("n_out,k_in,M", GEMM_SHAPES)
def test_gemm_against_fp64(env, wtype, n_out, k_in, M):
    torch, N, dev = env
    bits = _bf16_matrix(n_out, k_in, n_out * 5 + k_in)
    w32 = bf16_to_f32(bits)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((M, k_in)).astype(np.float32)
    xt = torch.from_numpy(x).to(dev)
    y = torch.full((M, n_out), float("nan"), dtype=torch.float32, device=dev)
    if wtype == "bf16":
        w_dev = torch.from_numpy(bits.view(np.int16)).to(dev)
        N.dar_op_gemm(0, _p(w_dev), None, n_out, k_in, _p(xt), M, _p(y), _sp(torch))
        w_ref = w32.astype(np.float64)
        sc = np.ones(n_out)
    else:
        codes, scale, w_ref, sc = _quantised(wtype, w32)
        w_dev = torch.from_numpy(codes).to(dev)
        s_dev = torch.from_numpy(scale).to(dev)
        N.dar_op_gemm(WT_CODES[wtype], _p(w_dev), _p(s_dev), n_out, k_in, _p(xt), M, _p(y), _sp(torch))
    got = y.cpu().numpy().astype(np.float64)
    want = (x.astype(np.float64) @ w_ref.T) * sc
    # inputs carried as bf16 hi + lo (relative error <= 2^-16), fp32 accumulation
    bound = 1e-5 * (np.abs(x.astype(np.float64)) @ np.abs(w_ref).T) * sc + 1e-30
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) / bound))


@pytest.mark.parametrize("n_q,n_kv,hd", [(4, 2, 64), (32, 8, 128), (8, 8, 128), (16, 2, 64)])
@pytest.mark.parametrize("pos", [0, 6, 63, 64, 200, 1022])
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("chunk", [0, 16])
def test_attention_against_fp64(env, n_q, n_kv, hd, pos, M, chunk):
    torch, N, dev = env
    max_len = 1024
    if pos + M > max_len:
        pytest.skip("past capacity")
    rng = np.random.default_rng(pos * 31 + M + hd)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((n_kv, max_len, hd)).astype(np.float32))
    vb = synth.f32_to_bf16_bits(rng.standard_normal((n_kv, max_len, hd)).astype(np.float32))
    q = (rng.standard_normal((M, n_q * hd)) * 0.5).astype(np.float32)
    K = torch.from_numpy(kb.view(np.int16)).to(dev)
    V = torch.from_numpy(vb.view(np.int16)).to(dev)
    qt = torch.from_numpy(q).to(dev)
    out = torch.full((M, n_q * hd), float("nan"), dtype=torch.float32, device=dev)
    N.dar_op_attention(_p(qt), _p(K), _p(V), n_q, n_kv, hd, max_len, pos, M, chunk, _p(out), _sp(torch))
    got = out.cpu().numpy().astype(np.float64).reshape(M, n_q, hd)
    k64 = bf16_to_f32(kb).astype(np.float64).transpose(1, 0, 2)     # [T, n_kv, hd]
    v64 = bf16_to_f32(vb).astype(np.float64).transpose(1, 0, 2)
    want = gqa_attention(q.astype(np.float64).reshape(M, n_q, hd), k64[:pos + M], v64[:pos + M],
                         np.arange(pos, pos + M))
    assert np.allclose(got, want, rtol=2e-5, atol=2e-6), float(np.max(np.abs(got - want)))
