"""Bytes a decode frame must move, and the pages' own bytes formula.

Decode at batch 1 is bound by streaming weights and the KV cache (tuna-fish
README, "Inference estimation": bytes per step = parameters without embeddings
plus the static KV buffer, turned into GB/s with it/s in "Inference
speedtest"). This module gives:

  * `pages_decode_elements` - the pages' formula, in elements;
  * `frame_bytes` - the algorithmic bytes one frame of this implementation must
    read: every weight matrix and norm the frame touches (the fast AR nine
    times), the codebook-0 head, the scales of quantised weights, the slow KV
    rows of the T positions the step attends to, and the fast AR's per-frame
    KV as read by its passes (pass k attends over k+1 fast positions). Embedding-row gathers
    (one row per step) are not counted.

Pure host arithmetic; no GPU, no library.
"""
from __future__ import annotations

GIB = 2 ** 30


def pages_decode_elements(p_slow, p_fast, n_slow, n_fast, c_kv, t_slow, t_fast, passes, batch=1):
    """Parameters plus static KV, in elements: (P_s + passes*P_f) + 2BLCT terms."""
    kv = 2 * batch * n_slow * c_kv * t_slow + 2 * batch * n_fast * c_kv * t_fast * passes
    return (p_slow + passes * p_fast) + kv


def layer_params(dims):
    d, F = dims.d_model, dims.ffn_dim
    mats = dims.qkv_rows * d + d * dims.q_width + 3 * F * d
    return mats, 2 * d          # (matrix entries, norm entries)


def layer_rows(dims):
    return dims.qkv_rows + dims.d_model + 2 * dims.ffn_dim + dims.d_model


def param_counts(dims, fast_head_rows=None):
    """Parameter counts per group (tables excluded except the tied head)."""
    mats, norms = layer_params(dims)
    out = {
        "slow_layers": dims.n_layers_slow * (mats + norms),
        "slow_final_norm": dims.d_model,
        "slow_head": dims.vocab_c0 * dims.d_model,
    }
    if dims.has_fast:
        rows = dims.vocab_res if fast_head_rows is None else fast_head_rows
        out["fast_layers"] = dims.n_layers_fast * (mats + norms)
        out["fast_final_norm"] = dims.d_model
        out["fast_head"] = rows * dims.d_model
    return out


def fast_params_wo_emb(dims, fast_head_rows=None):
    c = param_counts(dims, fast_head_rows)
    return c["fast_layers"] + c["fast_final_norm"] + c["fast_head"]


def kv_bytes_per_position(dims, kv_elem_bytes=2):
    return dims.n_layers_slow * 2 * dims.kv_width * kv_elem_bytes


def matrix_bytes(wtype, rows, entries):
    """Bytes of Linear matrices with `rows` rows and `entries` weights in all."""
    if wtype == "bf16":
        return 2 * entries
    if wtype in ("fp8", "int8"):  # one byte per weight + an fp32 scale per row
        return entries + 4 * rows
    if wtype == "int4":  # half a byte per weight + an fp32 scale per 128 weights of a row
        return entries // 2 + 4 * (entries // 128)
    raise ValueError(wtype)


def slow_weight_bytes(dims, wtype):
    mats, norms = layer_params(dims)
    L = dims.n_layers_slow
    w = matrix_bytes(wtype, L * layer_rows(dims), L * mats)
    return w + 2 * (L * norms + dims.d_model) + 2 * dims.vocab_c0 * dims.d_model


def fast_pass_bytes(dims, wtype):
    if not dims.has_fast:
        return 0
    mats, norms = layer_params(dims)
    L = dims.n_layers_fast
    head = dims.vocab_res * dims.d_model
    w = matrix_bytes(wtype, L * layer_rows(dims) + dims.vocab_res, L * mats + head)
    return w + 2 * (L * norms + dims.d_model)


def fast_kv_bytes(dims, kv_elem_bytes=2):
    """KV reads of the fast AR in one frame: pass k (1..R) reads k+1 positions."""
    if not dims.has_fast:
        return 0
    positions = sum(k + 1 for k in range(1, dims.n_res + 1))
    return positions * dims.n_layers_fast * 2 * dims.kv_width * kv_elem_bytes


def frame_bytes(dims, wtype, T, batch=1):
    """Algorithmic bytes of one decode step that attends over T slow positions."""
    passes = dims.n_res if dims.has_fast else 0
    return (slow_weight_bytes(dims, wtype) + passes * fast_pass_bytes(dims, wtype)
            + batch * (kv_bytes_per_position(dims) * T + fast_kv_bytes(dims)))


def run_bytes(dims, wtype, t_first, n_frames, batch=1):
    """Sum of frame_bytes over frames attending T = t_first .. t_first + n_frames - 1."""
    fixed = frame_bytes(dims, wtype, 0, batch)  # includes the fast KV
    t_sum = n_frames * t_first + n_frames * (n_frames - 1) // 2
    return n_frames * fixed + batch * kv_bytes_per_position(dims) * t_sum
