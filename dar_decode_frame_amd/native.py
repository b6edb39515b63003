"""ctypes binding of libdar.so (include/dar.h), same names as the C entry points.

Argument marshalling only: every computation happens in the HIP library.
Importing this module loads the library and raises if it has not been built
(`python -m dar_decode_frame_amd.build`); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdar.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "dar.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(HERE), "include", "dar_codec.h")]

DAR_OK = 0
DAR_E_INVAL = -1
DAR_E_STATE = -2
DAR_E_CAPACITY = -3
DAR_E_HIP = -4
DAR_E_WORKSPACE = -5
DAR_E_UNSUPPORTED = -6
DAR_WTYPE_BF16 = 0
DAR_WTYPE_FP8_E4M3_ROW = 1
DAR_WTYPE_INT8_ROW = 2
DAR_WTYPE_INT4_G128 = 3
WTYPES = {"bf16": 0, "fp8": DAR_WTYPE_FP8_E4M3_ROW, "int8": DAR_WTYPE_INT8_ROW, "int4": DAR_WTYPE_INT4_G128}
KIND_NAMES = {0: "qkv", 1: "attention", 2: "wo", 3: "w13", 4: "w2", 5: "head", 6: "other"}


class DarError(RuntimeError):
    def __init__(self, status, where, message=""):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_text(status)}) {message}".strip())


class dar_config(ctypes.Structure):
    _fields_ = [
        ("n_layers_slow", ctypes.c_int32),
        ("n_layers_fast", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("n_heads_q", ctypes.c_int32),
        ("n_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("ffn_dim", ctypes.c_int32),
        ("vocab_c0", ctypes.c_int32),
        ("vocab_res", ctypes.c_int32),
        ("n_res", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_double),
        ("max_len", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("wtype", ctypes.c_int32),
    ]


class dar_layer_weights(ctypes.Structure):
    _fields_ = [
        ("attn_norm", ctypes.c_void_p),
        ("wqkv", ctypes.c_void_p),
        ("wqkv_scale", ctypes.c_void_p),
        ("wo", ctypes.c_void_p),
        ("wo_scale", ctypes.c_void_p),
        ("ffn_norm", ctypes.c_void_p),
        ("w1", ctypes.c_void_p),
        ("w1_scale", ctypes.c_void_p),
        ("w3", ctypes.c_void_p),
        ("w3_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
    ]


class dar_sampling(ctypes.Structure):
    _fields_ = [
        ("temperature", ctypes.c_float),
        ("top_k", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("repetition_penalty", ctypes.c_float),
        ("repetition_window", ctypes.c_int32),
        ("uniforms", ctypes.c_void_p),
    ]


class dar_paging(ctypes.Structure):
    _fields_ = [
        ("page_len", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
    ]


class dar_weights(ctypes.Structure):
    _fields_ = [
        ("w0", ctypes.c_void_p),
        ("slow", ctypes.POINTER(dar_layer_weights)),
        ("slow_final_norm", ctypes.c_void_p),
        ("fast_emb", ctypes.POINTER(ctypes.c_void_p)),
        ("fast", ctypes.POINTER(dar_layer_weights)),
        ("fast_final_norm", ctypes.c_void_p),
        ("fast_head", ctypes.c_void_p),
        ("fast_head_scale", ctypes.c_void_p),
    ]


CODEC_MAX_BLOCKS = 8
CODEC_MAX_UNITS = 4


class dar_codec_config(ctypes.Structure):
    _fields_ = [
        ("n_codebooks", ctypes.c_int32),
        ("codebook_size", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("rates", ctypes.c_int32 * CODEC_MAX_BLOCKS),
        ("n_units", ctypes.c_int32),
        ("dilations", ctypes.c_int32 * CODEC_MAX_UNITS),
        ("kernel_size", ctypes.c_int32),
        ("max_frames", ctypes.c_int32),
    ]


class dar_codec_unit(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("alpha1", "w1", "b1", "alpha2", "w2", "b2")]


class dar_codec_block(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_void_p), ("up_w", ctypes.c_void_p), ("up_b", ctypes.c_void_p),
                ("units", dar_codec_unit * CODEC_MAX_UNITS)]


class dar_codec_weights(ctypes.Structure):
    _fields_ = [
        ("tables", ctypes.POINTER(ctypes.c_void_p)),
        ("in_w", ctypes.c_void_p),
        ("in_b", ctypes.c_void_p),
        ("blocks", ctypes.POINTER(dar_codec_block)),
        ("out_alpha", ctypes.c_void_p),
        ("out_w", ctypes.c_void_p),
        ("out_b", ctypes.c_void_p),
    ]


_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "dar_workspace_bytes": ([ctypes.POINTER(dar_config), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dar_create": ([ctypes.POINTER(dar_config), ctypes.POINTER(dar_weights), _VP, ctypes.c_size_t, _VP,
                    ctypes.POINTER(_VP)], ctypes.c_int),
    "dar_prefill": ([_VP, _I32, _VP, ctypes.POINTER(_I32), _VP, _VP, _VP], ctypes.c_int),
    "dar_workspace_bytes_paged": ([ctypes.POINTER(dar_config), ctypes.POINTER(dar_paging),
                                   ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dar_create_paged": ([ctypes.POINTER(dar_config), ctypes.POINTER(dar_paging), ctypes.POINTER(dar_weights), _VP,
                          ctypes.c_size_t, _VP, ctypes.POINTER(_VP)], ctypes.c_int),
    "dar_seq_add": ([_VP, _I32, _VP, _I32], ctypes.c_int),
    "dar_seq_remove": ([_VP, _I32], ctypes.c_int),
    "dar_pages_free": ([_VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_decode_frame": ([_VP, _VP, _VP, _VP], ctypes.c_int),
    "dar_destroy": ([_VP], ctypes.c_int),
    "dar_reset": ([_VP], ctypes.c_int),
    "dar_position": ([_VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_set_graph": ([_VP, _I32], ctypes.c_int),
    "dar_codes": ([_VP, _I32, _I32, _VP], ctypes.c_int),
    "dar_nonfinite": ([_VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_bytes_per_frame": ([ctypes.POINTER(dar_config), _I32, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "dar_quantize_fp8_rows": ([_VP, _I32, _I32, _VP, _VP, _VP], ctypes.c_int),
    "dar_quantize_int8_rows": ([_VP, _I32, _I32, _VP, _VP, _VP], ctypes.c_int),
    "dar_quantize_int4_groups": ([_VP, _I32, _I32, _VP, _VP, _VP], ctypes.c_int),
    "dar_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dar_last_error": ([_VP], ctypes.c_char_p),
    "dar_op_gemv": ([_I32, _VP, _VP, _I32, _I32, _VP, _I32, _VP, _VP], ctypes.c_int),
    "dar_op_gemm": ([_I32, _VP, _VP, _I32, _I32, _VP, _I32, _VP, _VP], ctypes.c_int),
    "dar_op_gemm_noalloc": ([_I32, _VP, _VP, _I32, _I32, _VP, _I32, _VP, _VP], ctypes.c_int),
    "dar_op_stream_read": ([_VP, ctypes.c_size_t, _I32, _VP, ctypes.POINTER(ctypes.c_float), _VP], ctypes.c_int),
    "dar_op_attention": ([_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP], ctypes.c_int),
    "dar_op_fp8_decode": ([_VP, _I32, _VP, _VP], ctypes.c_int),
    "dar_set_sampling": ([_VP, ctypes.POINTER(dar_sampling)], ctypes.c_int),
    "dar_op_sample": ([_VP, _I32, _I32, ctypes.POINTER(dar_sampling), _VP, _I32, _VP, _VP], ctypes.c_int),
    "dar_time_kind": ([_VP, _I32], ctypes.c_int),
    "dar_kind_time": ([_VP, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_profile_frame": ([_VP, _I32, _VP, _VP, _VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_codec_workspace_bytes": ([ctypes.POINTER(dar_codec_config), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dar_codec_create": ([ctypes.POINTER(dar_codec_config), ctypes.POINTER(dar_codec_weights), _VP, ctypes.c_size_t,
                          _VP, ctypes.POINTER(_VP)], ctypes.c_int),
    "dar_codec_decode": ([_VP, _VP, _I32, _VP], ctypes.c_int),
    "dar_codec_anomalies": ([_VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_codec_profile": ([_VP, _VP, _I32, _VP, _I32, _VP, _VP, ctypes.POINTER(_I32)], ctypes.c_int),
    "dar_codec_destroy": ([_VP], ctypes.c_int),
    "dar_codec_last_error": ([_VP], ctypes.c_char_p),
    "dar_codec_op_conv": ([_VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _I32, _I32, _I32, _VP, _I32, _VP, _VP],
                          ctypes.c_int),
    "dar_codec_op_resunit": ([_VP, _I32, _I32, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _I32, _VP, _VP],
                             ctypes.c_int),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dar_decode_frame_amd.build`")
    # The library and PyTorch must share one HIP runtime (device pointers and
    # streams cross between them). Loading torch first makes the library bind
    # to the runtime torch already holds instead of loading a second one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _status_text(status):
    try:
        return lib.dar_status_string(status).decode()
    except Exception:
        return "?"


def header_functions():
    """Names of every function declared in include/dar.h and include/dar_codec.h."""
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dar_\w+)\s*\(", text, flags=re.M)))


def _check(status, where, ctx=None):
    if status != DAR_OK:
        msg = lib.dar_last_error(ctx)
        raise DarError(status, where, msg.decode() if msg else "")
    return status


def make_config(dims, max_len, wtype="bf16", max_batch=1):
    """dar_config from any object with the DarDims attribute names."""
    return dar_config(
        dims.n_layers_slow, dims.n_layers_fast if dims.n_res > 0 else 0, dims.d_model, dims.n_heads_q,
        dims.n_heads_kv, dims.head_dim, dims.ffn_dim, dims.vocab_c0, dims.vocab_res, dims.n_res,
        dims.rms_eps, dims.rope_base, max_len, max_batch,
        WTYPES[wtype],
    )


# ---- the entry points, same names as in dar.h ------------------------------

def dar_workspace_bytes(cfg):
    out = ctypes.c_size_t(0)
    _check(lib.dar_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)), "dar_workspace_bytes")
    return out.value


def dar_create(cfg, weights, workspace_ptr, workspace_bytes, stream_ptr):
    ctx = ctypes.c_void_p(0)
    _check(lib.dar_create(ctypes.byref(cfg), ctypes.byref(weights), workspace_ptr, workspace_bytes, stream_ptr,
                          ctypes.byref(ctx)), "dar_create")
    return ctx


def dar_workspace_bytes_paged(cfg, paging):
    out = ctypes.c_size_t(0)
    _check(lib.dar_workspace_bytes_paged(ctypes.byref(cfg), ctypes.byref(paging), ctypes.byref(out)),
           "dar_workspace_bytes_paged")
    return out.value


def dar_create_paged(cfg, paging, weights, workspace_ptr, workspace_bytes, stream_ptr):
    ctx = ctypes.c_void_p(0)
    _check(lib.dar_create_paged(ctypes.byref(cfg), ctypes.byref(paging), ctypes.byref(weights), workspace_ptr,
                                workspace_bytes, stream_ptr, ctypes.byref(ctx)), "dar_create_paged")
    return ctx


def dar_seq_add(ctx, slot, tokens_ptr, length):
    return _check(lib.dar_seq_add(ctx, slot, tokens_ptr, length), "dar_seq_add", ctx)


def dar_seq_remove(ctx, slot):
    return _check(lib.dar_seq_remove(ctx, slot), "dar_seq_remove", ctx)


def dar_pages_free(ctx):
    out = ctypes.c_int32(0)
    _check(lib.dar_pages_free(ctx, ctypes.byref(out)), "dar_pages_free", ctx)
    return out.value


def dar_prefill(ctx, batch, tokens_ptr, lens, forced_ptr=None, codes_out_ptr=None, logits_out_ptr=None):
    lens_arr = (ctypes.c_int32 * len(lens))(*lens)
    return _check(lib.dar_prefill(ctx, batch, tokens_ptr, lens_arr, forced_ptr, codes_out_ptr, logits_out_ptr),
                  "dar_prefill", ctx)


def dar_decode_frame(ctx, forced_ptr=None, codes_out_ptr=None, logits_out_ptr=None):
    return _check(lib.dar_decode_frame(ctx, forced_ptr, codes_out_ptr, logits_out_ptr), "dar_decode_frame", ctx)


def dar_destroy(ctx):
    return _check(lib.dar_destroy(ctx), "dar_destroy")


def dar_reset(ctx):
    return _check(lib.dar_reset(ctx), "dar_reset", ctx)


def dar_position(ctx, max_batch=1):
    out = (ctypes.c_int32 * max_batch)()
    _check(lib.dar_position(ctx, out), "dar_position", ctx)
    return list(out)


def dar_set_graph(ctx, enable):
    return _check(lib.dar_set_graph(ctx, 1 if enable else 0), "dar_set_graph", ctx)


def dar_codes(ctx, first, count, dst_ptr):
    return _check(lib.dar_codes(ctx, first, count, dst_ptr), "dar_codes", ctx)


def dar_nonfinite(ctx):
    out = ctypes.c_int32(0)
    _check(lib.dar_nonfinite(ctx, ctypes.byref(out)), "dar_nonfinite", ctx)
    return out.value


def dar_bytes_per_frame(cfg, T):
    out = ctypes.c_double(0)
    _check(lib.dar_bytes_per_frame(ctypes.byref(cfg), T, ctypes.byref(out)), "dar_bytes_per_frame")
    return out.value


def dar_quantize_fp8_rows(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr):
    return _check(lib.dar_quantize_fp8_rows(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr), "dar_quantize_fp8_rows")


def dar_quantize_int8_rows(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr):
    return _check(lib.dar_quantize_int8_rows(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr), "dar_quantize_int8_rows")


def dar_quantize_int4_groups(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr):
    return _check(lib.dar_quantize_int4_groups(w_ptr, rows, cols, q_ptr, scale_ptr, stream_ptr),
                  "dar_quantize_int4_groups")


def dar_status_string(status):
    return lib.dar_status_string(status).decode()


def dar_last_error(ctx=None):
    return lib.dar_last_error(ctx).decode()


def dar_op_gemv(wtype, w_ptr, scale_ptr, rows, cols, x_ptr, M, y_ptr, stream_ptr):
    return _check(lib.dar_op_gemv(wtype, w_ptr, scale_ptr, rows, cols, x_ptr, M, y_ptr, stream_ptr), "dar_op_gemv")


def dar_op_attention(q_ptr, k_ptr, v_ptr, n_heads_q, n_heads_kv, head_dim, max_len, pos, M, chunk, out_ptr,
                     stream_ptr):
    return _check(lib.dar_op_attention(q_ptr, k_ptr, v_ptr, n_heads_q, n_heads_kv, head_dim, max_len, pos, M, chunk,
                                       out_ptr, stream_ptr), "dar_op_attention")


def dar_op_gemm(wtype, w_ptr, scale_ptr, N, K, x_ptr, M, y_ptr, stream_ptr):
    return _check(lib.dar_op_gemm(wtype, w_ptr, scale_ptr, N, K, x_ptr, M, y_ptr, stream_ptr), "dar_op_gemm")


def dar_op_gemm_noalloc(wtype, w_ptr, scale_ptr, N, K, x_ptr, M, y_ptr, stream_ptr):
    return _check(lib.dar_op_gemm_noalloc(wtype, w_ptr, scale_ptr, N, K, x_ptr, M, y_ptr, stream_ptr),
                  "dar_op_gemm_noalloc")


def dar_op_stream_read(src_ptr, nbytes, iters, sink_ptr, stream_ptr):
    """Mean milliseconds per plain read of nbytes at src (see dar.h)."""
    ms = ctypes.c_float(0.0)
    _check(lib.dar_op_stream_read(src_ptr, nbytes, iters, sink_ptr, ctypes.byref(ms), stream_ptr),
           "dar_op_stream_read")
    return ms.value


def dar_op_fp8_decode(codes_ptr, n, out_ptr, stream_ptr):
    return _check(lib.dar_op_fp8_decode(codes_ptr, n, out_ptr, stream_ptr), "dar_op_fp8_decode")


def make_sampling(temperature, top_k, top_p, repetition_penalty, repetition_window, uniforms_ptr):
    return dar_sampling(temperature, top_k, top_p, repetition_penalty, repetition_window, uniforms_ptr)


def dar_set_sampling(ctx, sampling):
    """sampling: a dar_sampling, or None for greedy argmax."""
    return _check(lib.dar_set_sampling(ctx, ctypes.byref(sampling) if sampling is not None else None),
                  "dar_set_sampling", ctx)


def dar_op_sample(logits_ptr, rows, V, sampling, history_ptr, n_hist, codes_ptr, stream_ptr):
    return _check(lib.dar_op_sample(logits_ptr, rows, V, ctypes.byref(sampling), history_ptr, n_hist, codes_ptr,
                                    stream_ptr), "dar_op_sample")


def dar_time_kind(ctx, kind):
    return _check(lib.dar_time_kind(ctx, kind), "dar_time_kind", ctx)


def dar_kind_time(ctx):
    """(summed ms, launches) of the launches timed since dar_time_kind or the last read."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(lib.dar_kind_time(ctx, ctypes.byref(ms), ctypes.byref(n)), "dar_kind_time", ctx)
    return ms.value, n.value


def dar_profile_frame(ctx, cap=4096):
    """Per launch: (ms, kind, layer tag)."""
    ms = (ctypes.c_float * cap)()
    kind = (ctypes.c_int32 * cap)()
    layer = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32(0)
    _check(lib.dar_profile_frame(ctx, cap, ms, kind, layer, ctypes.byref(n)), "dar_profile_frame", ctx)
    return [(float(ms[i]), int(kind[i]), int(layer[i])) for i in range(n.value)]


# ---- codec (include/dar_codec.h)

def _check_codec(status, where, ctx=None):
    if status != DAR_OK:
        msg = lib.dar_codec_last_error(ctx)
        raise DarError(status, where, msg.decode() if msg else "")
    return status


def make_codec_config(dims, max_frames):
    """dar_codec_config from any object with the CodecDims attribute names."""
    c = dar_codec_config()
    c.n_codebooks = dims.n_codebooks
    c.codebook_size = dims.codebook_size
    c.latent_dim = dims.latent_dim
    c.channels = dims.channels
    c.n_blocks = len(dims.rates)
    for i, r in enumerate(dims.rates):
        c.rates[i] = r
    c.n_units = len(dims.dilations)
    for i, d in enumerate(dims.dilations):
        c.dilations[i] = d
    c.kernel_size = dims.kernel
    c.max_frames = max_frames
    return c


def dar_codec_workspace_bytes(cfg):
    out = ctypes.c_size_t(0)
    _check_codec(lib.dar_codec_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)), "dar_codec_workspace_bytes")
    return out.value


def dar_codec_create(cfg, weights, ws_ptr, ws_bytes, stream_ptr):
    ctx = ctypes.c_void_p(0)
    _check_codec(lib.dar_codec_create(ctypes.byref(cfg), ctypes.byref(weights), ws_ptr, ws_bytes, stream_ptr,
                                      ctypes.byref(ctx)), "dar_codec_create")
    return ctx


def dar_codec_decode(ctx, codes_ptr, frames, audio_ptr):
    return _check_codec(lib.dar_codec_decode(ctx, codes_ptr, frames, audio_ptr), "dar_codec_decode", ctx)


def dar_codec_anomalies(ctx):
    out = ctypes.c_int32(0)
    _check_codec(lib.dar_codec_anomalies(ctx, ctypes.byref(out)), "dar_codec_anomalies", ctx)
    return out.value


def dar_codec_profile(ctx, codes_ptr, frames, audio_ptr, cap=256):
    """Per launch of one decode: (ms, tag)."""
    ms = (ctypes.c_float * cap)()
    tag = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32(0)
    _check_codec(lib.dar_codec_profile(ctx, codes_ptr, frames, audio_ptr, cap, ms, tag, ctypes.byref(n)),
                 "dar_codec_profile", ctx)
    return [(float(ms[i]), int(tag[i])) for i in range(n.value)]


def dar_codec_destroy(ctx):
    return _check_codec(lib.dar_codec_destroy(ctx), "dar_codec_destroy")


def dar_codec_op_conv(x_ptr, x_bf16, alpha_ptr, T, Cin, Cout, w_ptr, b_ptr, taps, dilation, stride, res_ptr,
                      tanh_out, y_ptr, stream_ptr):
    return _check_codec(lib.dar_codec_op_conv(x_ptr, x_bf16, alpha_ptr, T, Cin, Cout, w_ptr, b_ptr, taps, dilation,
                                              stride, res_ptr, tanh_out, y_ptr, stream_ptr), "dar_codec_op_conv")


def dar_codec_op_resunit(x_ptr, T, C, alpha1_ptr, w1_ptr, b1_ptr, taps, dilation, alpha2_ptr, w2_ptr, b2_ptr, fused,
                         y_ptr, stream_ptr):
    return _check_codec(lib.dar_codec_op_resunit(x_ptr, T, C, alpha1_ptr, w1_ptr, b1_ptr, taps, dilation, alpha2_ptr,
                                                 w2_ptr, b2_ptr, fused, y_ptr, stream_ptr), "dar_codec_op_resunit")
