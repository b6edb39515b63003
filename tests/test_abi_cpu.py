"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before touching HIP.

dar_bytes_per_frame must agree with the host bytes model, which is itself
pinned to the pages' numbers (tests/test_bytes_model.py)."""
import ctypes

import numpy as np

import pytest

from dar_decode_frame_amd import bytes_model as bm
import synth
from synth import DIMS


@pytest.fixture(scope="module")
def N():
    from dar_decode_frame_amd import native
    return native


def test_every_declared_symbol_is_exported(N):
    names = N.header_functions()
    assert len(names) >= 18
    for name in names:
        assert hasattr(N.lib, name), name
        assert name in N._SIGS, f"binding misses {name}"


@pytest.mark.parametrize("dname,max_len", [("tiny", 32), ("s2pro_slow", 1024), ("s2pro_dual", 1024)])
def test_workspace_bytes_cover_kv(N, dname, max_len):
    d = DIMS[dname]
    n = N.dar_workspace_bytes(N.make_config(d, max_len))
    kv = 2 * d.n_layers_slow * d.n_heads_kv * max_len * d.head_dim * 2
    # beyond the slow KV cache: decode activations and the prefill block's
    # scratch (128 rows of every activation, GEMM and attention partial sums)
    assert n >= kv and n < kv + 160 * 2 ** 20


@pytest.mark.parametrize("dname,wtype", [("tiny", "bf16"), ("tiny", "fp8"), ("tiny", "int8"), ("tiny", "int4"),
                                         ("s2pro_slow", "bf16"), ("s2pro_dual", "bf16"), ("s2pro_dual", "fp8"),
                                         ("s2pro_dual", "int8"), ("s2pro_dual", "int4")])
@pytest.mark.parametrize("T", [0, 1, 129, 1024])
def test_bytes_per_frame_matches_host_model(N, dname, wtype, T):
    d = DIMS[dname]
    got = N.dar_bytes_per_frame(N.make_config(d, 1024, wtype), T)
    assert got == float(bm.frame_bytes(d, wtype, T))


def _cfg(N, **kw):
    c = N.make_config(DIMS["tiny"], 32)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, -6), ("n_heads_kv", 3, -1), ("d_model", 200, -6), ("max_batch", 65, -6), ("max_batch", 0, -1),
    ("max_len", 1, -1), ("rms_eps", 0.0, -1), ("rope_base", 1.0, -1), ("wtype", 7, -1),
    ("n_res", 16, -6), ("n_layers_slow", 0, -1), ("vocab_c0", 0, -1),
])
def test_config_validation(N, field, value, status):
    c = _cfg(N, **{field: value})
    out = ctypes.c_size_t(0)
    assert N.lib.dar_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == status
    assert N.dar_last_error(None)


def test_create_rejects_before_hip(N):
    c = _cfg(N)
    w = N.dar_weights()
    ctx = ctypes.c_void_p(0)
    need = N.dar_workspace_bytes(c)
    # NULL weights pointers
    assert N.lib.dar_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(1 << 20), need, None,
                            ctypes.byref(ctx)) == N.DAR_E_INVAL
    # misaligned workspace
    assert N.lib.dar_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p((1 << 20) + 8), need, None,
                            ctypes.byref(ctx)) == N.DAR_E_INVAL
    # workspace too small
    assert N.lib.dar_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(1 << 20), need - 1, None,
                            ctypes.byref(ctx)) == N.DAR_E_WORKSPACE
    assert ctx.value is None
    # misaligned weight pointers are caught too
    layers = (N.dar_layer_weights * 2)()
    for L in layers:
        for f, _ in N.dar_layer_weights._fields_:
            setattr(L, f, 4096 + 2)
    w.w0 = 4096
    w.slow = layers
    w.slow_final_norm = 4096
    assert N.lib.dar_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(1 << 20), need, None,
                            ctypes.byref(ctx)) == N.DAR_E_INVAL


def test_null_context_and_ops_reject(N):
    assert N.lib.dar_prefill(None, 1, None, None, None, None, None) == N.DAR_E_INVAL
    assert N.lib.dar_decode_frame(None, None, None, None) == N.DAR_E_INVAL
    assert N.lib.dar_reset(None) == N.DAR_E_INVAL
    assert N.lib.dar_destroy(None) == N.DAR_OK
    assert N.lib.dar_op_gemv(0, None, None, 4, 256, None, 1, None, None) == N.DAR_E_INVAL
    assert N.lib.dar_op_gemv(0, ctypes.c_void_p(4096), None, 4, 300, ctypes.c_void_p(4096), 1,
                             ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
    for wq in (1, 2, 3):  # fp8, int8 and int4 weights need their scales
        assert N.lib.dar_op_gemv(wq, ctypes.c_void_p(4096), None, 4, 256, ctypes.c_void_p(4096), 1,
                                 ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
        assert N.lib.dar_op_gemm(wq, ctypes.c_void_p(4096), None, 4, 256, ctypes.c_void_p(4096), 1,
                                 ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_gemv(4, ctypes.c_void_p(4096), ctypes.c_void_p(4096), 4, 256, ctypes.c_void_p(4096), 1,
                             ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_attention(None, None, None, 4, 2, 64, 16, 0, 1, 0, None, None) == N.DAR_E_INVAL
    # the reference read: 16-byte aligned source, a multiple of 16 bytes, at least one read, all pointers
    ms = ctypes.c_float(0)
    src, sink = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert N.lib.dar_op_stream_read(src, 100, 1, sink, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(src, 0, 1, sink, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(src, 1024, 0, sink, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(ctypes.c_void_p(4100), 1024, 1, sink, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(None, 1024, 1, sink, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(src, 1024, 1, None, ctypes.byref(ms), None) == N.DAR_E_INVAL
    assert N.lib.dar_op_stream_read(src, 1024, 1, sink, None, None) == N.DAR_E_INVAL
    assert N.lib.dar_quantize_fp8_rows(ctypes.c_void_p(4096), 4, 24, ctypes.c_void_p(4096),
                                       ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
    assert N.lib.dar_quantize_int8_rows(ctypes.c_void_p(4096), 4, 24, ctypes.c_void_p(4096),
                                        ctypes.c_void_p(4096), None) == N.DAR_E_INVAL
    for cols in (64, 200):  # int4 groups are 128 columns
        assert N.lib.dar_quantize_int4_groups(ctypes.c_void_p(4096), 4, cols, ctypes.c_void_p(4096),
                                              ctypes.c_void_p(4096), None) == N.DAR_E_INVAL


def test_status_strings(N):
    for s in range(-6, 1):
        assert N.dar_status_string(s) not in ("", "unknown status")
    assert N.dar_status_string(-99) == "unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("temperature", 0.0, -1), ("temperature", float("inf"), -1), ("top_k", 0, -1), ("top_k", 257, -6),
    ("top_p", 0.0, -1), ("top_p", 1.5, -1), ("repetition_penalty", 0.5, -1), ("repetition_window", -1, -1),
    ("repetition_window", 65, -6), ("uniforms", None, -1),
])
def test_sampling_argument_checks(N, field, value, status):
    """Checked on the host before any launch (no GPU needed)."""
    s = N.make_sampling(0.8, 50, 0.9, 1.2, 16, 4096)
    setattr(s, field, value)
    p = ctypes.c_void_p(4096)
    assert N.lib.dar_op_sample(p, 4, 1024, ctypes.byref(s), p, 4, p, None) == status
    assert N.lib.dar_set_sampling(None, ctypes.byref(s)) == N.DAR_E_INVAL


def test_sampling_vocabulary_limit(N):
    s = N.make_sampling(0.8, 50, 0.9, 1.2, 16, 4096)
    p = ctypes.c_void_p(4096)
    assert N.lib.dar_op_sample(p, 4, 8193, ctypes.byref(s), p, 4, p, None) == N.DAR_E_UNSUPPORTED
    assert N.lib.dar_op_sample(p, 0, 1024, ctypes.byref(s), p, 4, p, None) == N.DAR_E_INVAL
    assert N.lib.dar_op_sample(p, 4, 1024, ctypes.byref(s), None, 4, p, None) == N.DAR_E_INVAL


@pytest.mark.parametrize("page_len,n_pages,max_batch,max_len,status", [
    (64, 2, 2, 32, 0), (256, 40, 16, 4096, 0),
    (96, 8, 2, 256, -1), (32, 8, 2, 256, -1), (64, 1, 2, 256, -1),   # not a power of two, below 64, no usable page
    (64, 8, 1, 256, -6),                                              # paged contexts use the many-row path
    (64, 80, 2, 64 * 65, -6),                                         # 65 pages per sequence
])
def test_paging_validation(N, page_len, n_pages, max_batch, max_len, status):
    c = _cfg(N, max_batch=max_batch, max_len=max_len)
    pg = N.dar_paging(page_len, n_pages)
    out = ctypes.c_size_t(0)
    assert N.lib.dar_workspace_bytes_paged(ctypes.byref(c), ctypes.byref(pg), ctypes.byref(out)) == status
    ctx = ctypes.c_void_p(0)
    if status != 0:
        assert N.dar_last_error(None)
        # create rejects the same arguments before any HIP call
        w = N.dar_weights()
        assert N.lib.dar_create_paged(ctypes.byref(c), ctypes.byref(pg), ctypes.byref(w), ctypes.c_void_p(256),
                                      out.value or 1 << 30, None, ctypes.byref(ctx)) == status
        assert not ctx.value


def test_paged_workspace_holds_the_pool(N):
    # the slow KV is the page pool instead of max_batch full-length caches
    d = DIMS["s2pro_dual"]
    c = N.make_config(d, 4096, max_batch=16)
    full = N.dar_workspace_bytes(c)
    page_bytes = 2 * d.n_layers_slow * d.n_heads_kv * 256 * d.head_dim * 2
    for n_pages in (17, 65):
        paged = N.dar_workspace_bytes_paged(c, N.dar_paging(256, n_pages))
        kv_full = 2 * d.n_layers_slow * 16 * d.n_heads_kv * 4096 * d.head_dim * 2
        assert paged - (full - kv_full) >= n_pages * page_bytes
        assert paged - (full - kv_full) < n_pages * page_bytes + 2 ** 20


def test_paged_calls_reject_without_context(N):
    n = ctypes.c_int32(0)
    assert N.lib.dar_seq_add(None, 0, ctypes.c_void_p(256), 4) == N.DAR_E_INVAL
    assert N.lib.dar_seq_remove(None, 0) == N.DAR_E_INVAL
    assert N.lib.dar_pages_free(None, ctypes.byref(n)) == N.DAR_E_INVAL


def _codec_cfg(N, **kw):
    c = N.make_codec_config(synth.CODEC_DIMS["tiny_codec"], 64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_codec_workspace_holds_weights_and_activations(N):
    d = synth.CODEC_DIMS["s2pro_codec"]
    n = N.dar_codec_workspace_bytes(N.make_codec_config(d, 167))
    params = sum(int(np.prod(shape)) for name, shape, _, _ in synth.codec_tensor_specs(d)
                 if name.endswith((".w", ".w1", ".w2")))
    act = 167 * d.hop * d.widths[-1]  # the widest activation: 2048 samples x 96 channels per frame
    # bf16 weights; two fp32 activation buffers; bf16 hidden rows and two bf16 operand buffers
    assert n >= 2 * params + 2 * 4 * act + 3 * 2 * act
    assert n < 2 * params + 2 * 4 * act + 3 * 2 * act + 64 * 2 ** 20


@pytest.mark.parametrize("field,value", [
    ("n_codebooks", 0), ("n_codebooks", 33), ("latent_dim", 48), ("channels", 100), ("n_blocks", 0),
    ("n_blocks", 9), ("kernel_size", 4), ("kernel_size", 9), ("n_units", 0), ("max_frames", 0),
])
def test_codec_config_validation(N, field, value):
    c = _codec_cfg(N, **{field: value})
    out = ctypes.c_size_t(0)
    assert N.lib.dar_codec_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == N.DAR_E_INVAL
    assert N.lib.dar_codec_last_error(None)


def test_codec_rates_and_dilations_checked(N):
    c = _codec_cfg(N)
    c.rates[1] = 3                        # odd stride
    out = ctypes.c_size_t(0)
    assert N.lib.dar_codec_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == N.DAR_E_INVAL
    c = _codec_cfg(N)
    c.dilations[2] = 11                   # 3 * 11 > 32 positions of reach
    assert N.lib.dar_codec_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == N.DAR_E_INVAL


def test_codec_create_rejects_before_hip(N):
    c = _codec_cfg(N)
    need = N.dar_codec_workspace_bytes(c)
    w = N.dar_codec_weights()
    ctx = ctypes.c_void_p(0)
    assert N.lib.dar_codec_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(1 << 20), need, None,
                                  ctypes.byref(ctx)) == N.DAR_E_INVAL
    assert N.lib.dar_codec_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(1 << 20), need - 1, None,
                                  ctypes.byref(ctx)) == N.DAR_E_WORKSPACE
    assert N.lib.dar_codec_decode(None, None, 1, None) == N.DAR_E_INVAL


def test_codec_ops_reject_bad_arguments_before_hip(N):
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    # one residual unit: the one-launch kernel needs a width a tile spans and y != x
    args = dict(T=100, C=96, taps=7, dilation=3, fused=1)

    def unit(**kw):
        a = dict(args, **kw)
        return N.lib.dar_codec_op_resunit(fake, a["T"], a["C"], fake, fake, fake, a["taps"], a["dilation"], fake,
                                          fake, fake, a["fused"], ctypes.c_void_p(2 << 20), None)

    assert unit(C=192) == N.DAR_E_INVAL            # no one-launch tile at 192 channels
    assert b"one-launch" in N.lib.dar_codec_last_error(None)
    assert unit(C=100, fused=0) == N.DAR_E_INVAL   # not a multiple of 32
    assert unit(taps=4) == N.DAR_E_INVAL           # even kernel
    assert unit(dilation=11) == N.DAR_E_INVAL      # 3 * 11 > 32 rows of reach
    assert unit(T=0) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_resunit(fake, 100, 96, fake, fake, fake, 7, 1, fake, fake, fake, 1, fake,
                                      None) == N.DAR_E_INVAL  # in place
    # one convolution: widths, taps and strides
    assert N.lib.dar_codec_op_conv(fake, 0, fake, 10, 48, 64, fake, fake, 7, 1, 0, None, 0, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 0, fake, 10, 64, 64, fake, fake, 7, 1, 3, None, 0, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, fake, 10, 64, 64, fake, fake, 7, 1, 0, None, 0, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 0, None, 10, 64, 1, fake, fake, 7, 1, 0, None, 1, fake, None) == N.DAR_E_INVAL
    # the output convolution: bf16 operand without alpha or fp32 rows with it; odd taps <= 7; tanh; no residual
    assert N.lib.dar_codec_op_conv(fake, 1, fake, 10, 64, 1, fake, fake, 7, 1, 0, None, 1, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, None, 10, 64, 1, fake, fake, 9, 1, 0, None, 1, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, None, 10, 64, 1, fake, fake, 6, 1, 0, None, 1, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, None, 10, 48, 1, fake, fake, 7, 1, 0, None, 1, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, None, 10, 64, 1, fake, fake, 7, 1, 0, None, 0, fake, None) == N.DAR_E_INVAL
    assert N.lib.dar_codec_op_conv(fake, 1, None, 10, 64, 1, fake, fake, 7, 1, 0, fake, 1, fake, None) == N.DAR_E_INVAL
