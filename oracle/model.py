"""The Dual-AR (RQ-Transformer) decode, written out plainly (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, and where the pages say so:
  * Dual-AR frame: a slow AR runs along time and predicts codebook 0; a fast AR
    runs along depth and emits the nine residual codebooks of the same frame,
    one after another (groxaxo fork README, architecture paragraph; tuna-fish
    README intro: "slowAR decode + fastAR loop"; its "Inference estimation"
    charges the fast weights nine times per frame against a fast KV of length
    10).
  * The block is a decoder-only LLaMA-style layer with rotary embeddings and
    grouped-query attention (pyshine fish-speech tour, "Why You Need This"),
    pre-RMSNorm, SwiGLU FFN, no biases.
  * The slow AR's input table is tied to its codebook-0 head (tuna-fish README,
    "training estimation": slow AR "tied emb" parameters).
  * Greedy decoding: each codebook is the first index of the largest logit.

Readings where the pages leave a step open (each also listed in the design doc):
  * The slow AR consumes only the previous frame's codebook-0 id per step.
  * RoPE pairs element i with i + hd/2 (rotate-half); angle p * base^(-2i/hd)
    is formed in fp64, cos/sin rounded to the working precision. Slow positions
    count from 0 at the first prompt token; fast positions restart at 0 in
    every frame.
  * Query head h reads KV head floor(h / (n_q / n_kv)).
  * The fast AR sees the sequence [h_t, E0[c0], E1[c1], ..., E_{R-1}[c_{R-1}]]
    at fast positions 0..R, where h_t is the slow AR's final-normed hidden
    vector (the one that also feeds the codebook-0 head); the output at fast
    position k >= 1 goes through the fast final norm and the shared fast head
    to give codebook k.
  * Teacher forcing: a forced frame replaces the committed codes (what the next
    steps consume); logits and argmax codes are still the model's own.

Precision: `dt` (np.float32 by default, np.float64 for cross-checks). Weights
are the canonical bf16 values (or, for fp8, s * dec(q)), held in `dt`. The KV
caches hold activations, whose dtype the s2-pro-fp8 model card ("What is
this?") gives as bfloat16: cached keys (after RoPE) and values are rounded to
bf16 (nearest even) when written, unless kv="fp32". Queries, scores, softmax,
the residual stream and every matrix product stay in `dt`.
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, quantize_rows
from .int4 import dequantize_int4, quantize_int4_groups
from .int8 import quantize_int8_rows


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each entry, returned in x's dtype.

    fp64 inputs are first rounded to fp32 (the precision the KV values are
    produced in); NaN stays NaN.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(f), f, out)
    return out.astype(np.asarray(x).dtype, copy=False)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=dt)
    return (x / np.sqrt(ms + dt.type(eps))) * g.astype(dt)


def silu(a: np.ndarray) -> np.ndarray:
    """a * sigmoid(a) = a / (1 + exp(-a))."""
    one = a.dtype.type(1.0)
    return a / (one + np.exp(-a))


def rope_cos_sin(positions, head_dim: int, base: float, dt=np.float32):
    """cos/sin of theta[p, i] = p * base^(-2i/hd), i < hd/2; angles in fp64."""
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    theta = pos[:, None] * inv_freq[None, :]
    return np.cos(theta).astype(dt), np.sin(theta).astype(dt)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (v_i, v_{i+hd/2}) by theta_i. cos/sin broadcast against v[..., :hd/2]."""
    half = v.shape[-1] // 2
    a = v[..., :half]
    b = v[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention of a block of queries against cached keys.

    q [n, n_q, hd] at absolute positions q_pos [n]; k, v [T, n_kv, hd] for
    positions 0..T-1. Query i sees keys j <= q_pos[i]. Returns [n, n_q, hd].
    """
    n, n_q, hd = q.shape
    T, n_kv, _ = k.shape
    g = n_q // n_kv
    dt = q.dtype
    scale = dt.type(1.0 / np.sqrt(hd))
    mask = np.arange(T)[None, :] <= np.asarray(q_pos)[:, None]          # [n, T]
    out = np.empty_like(q)
    for h in range(n_q):
        kv = h // g
        s = (q[:, h, :] @ k[:, kv, :].T) * scale                          # [n, T]
        s = np.where(mask, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def greedy_argmax(logits: np.ndarray) -> int:
    """First index of the maximum; NaN counts as -inf."""
    clean = np.where(np.isnan(logits), -np.inf, logits)
    return int(np.argmax(clean))


class Linear:
    """y = W x for W [out][in]; the quantised forms keep (dec(q), s) and return s * (dec(q) x)."""

    def __init__(self, w: np.ndarray, scale: np.ndarray | None = None):
        self.w = w
        self.scale = scale

    def __call__(self, x: np.ndarray) -> np.ndarray:
        y = x @ self.w.T
        if self.scale is not None:
            y = y * self.scale
        return y


class _Layer:
    def __init__(self, get, get_lin, prefix):
        self.attn_norm = get(f"{prefix}.attn_norm")
        self.wqkv = get_lin(f"{prefix}.wqkv")
        self.wo = get_lin(f"{prefix}.wo")
        self.ffn_norm = get(f"{prefix}.ffn_norm")
        self.w1 = get_lin(f"{prefix}.w1")
        self.w3 = get_lin(f"{prefix}.w3")
        self.w2 = get_lin(f"{prefix}.w2")


class OracleModel:
    """Weights of one Dual-AR model held in the oracle's working precision.

    tensors: {name: uint16 bf16 bits} in the canonical list's names.
    wtype "fp8": every Linear matrix (the ones named *.wqkv, *.wo, *.w1, *.w3,
    *.w2 and fast.head) is quantised per row with the oracle's quantiser and
    used as s * dec(q); tables and norm gains stay bf16. wtype "int8": the same
    matrices quantised per row to int8 (oracle/int8.py), used as s * q.
    wtype "int4": the same matrices quantised to int4 in groups of 128 columns
    (oracle/int4.py), used as the dequantised s_g * q.
    """

    def __init__(self, dims, tensors: dict, wtype: str = "bf16", dt=np.float32, drop_source: bool = False,
                 kv: str = "bf16"):
        if wtype not in ("bf16", "fp8", "int8", "int4"):
            raise ValueError(wtype)
        if kv not in ("bf16", "fp32"):
            raise ValueError(kv)
        self.dims = dims
        self.wtype = wtype
        self.dt = dt
        self.kv_bf16 = kv == "bf16"
        self.quant = {}  # name -> (codes, row scales) of every quantised matrix

        def get(name):
            return bf16_to_f32(tensors[name]).astype(dt, copy=False)

        def get_lin(name):
            w = bf16_to_f32(tensors[name])
            if wtype == "bf16":
                out = Linear(w.astype(dt, copy=False))
            elif wtype == "int8":
                codes, scale = quantize_int8_rows(w)
                self.quant[name] = (codes, scale)
                out = Linear(codes.astype(dt), scale.astype(dt))
            elif wtype == "int4":
                codes, scale = quantize_int4_groups(w)
                self.quant[name] = (codes, scale)
                out = Linear(dequantize_int4(codes, scale).astype(dt, copy=False))
            else:
                codes, scale = quantize_rows(w)
                self.quant[name] = (codes, scale)
                out = Linear(e4m3_decode(codes).astype(dt, copy=False), scale.astype(dt))
            if drop_source:
                tensors.pop(name, None)
            return out

        self.w0 = get("w0")
        self.slow = [_Layer(get, get_lin, f"slow.{i}") for i in range(dims.n_layers_slow)]
        self.slow_final_norm = get("slow.final_norm")
        self.fast = []
        if dims.has_fast:
            self.fast_emb = [get(f"fast.emb.{k}") for k in range(dims.n_res)]
            self.fast = [_Layer(get, get_lin, f"fast.{i}") for i in range(dims.n_layers_fast)]
            self.fast_final_norm = get("fast.final_norm")
            self.fast_head = get_lin("fast.head")

    # ---- one block over new positions, reading and extending a KV cache ----
    def block(self, layer: _Layer, x: np.ndarray, p0: int, cache_k: np.ndarray, cache_v: np.ndarray):
        """x [n, d] at positions p0..p0+n-1; cache_k/v [max_len, n_kv, hd] (written in place)."""
        d = self.dims
        n = x.shape[0]
        qw, kvw, hd = d.q_width, d.kv_width, d.head_dim
        h = rmsnorm(x, layer.attn_norm, d.rms_eps)
        qkv = layer.wqkv(h)
        q = qkv[:, :qw].reshape(n, d.n_heads_q, hd)
        k = qkv[:, qw:qw + kvw].reshape(n, d.n_heads_kv, hd)
        v = qkv[:, qw + kvw:].reshape(n, d.n_heads_kv, hd)
        pos = np.arange(p0, p0 + n)
        cos, sin = rope_cos_sin(pos, hd, d.rope_base, self.dt)
        q = apply_rope(q, cos[:, None, :], sin[:, None, :])
        k = apply_rope(k, cos[:, None, :], sin[:, None, :])
        cache_k[p0:p0 + n] = round_bf16(k) if self.kv_bf16 else k
        cache_v[p0:p0 + n] = round_bf16(v) if self.kv_bf16 else v
        o = gqa_attention(q, cache_k[:p0 + n], cache_v[:p0 + n], pos)
        x = x + layer.wo(o.reshape(n, qw))
        h2 = rmsnorm(x, layer.ffn_norm, d.rms_eps)
        x = x + layer.w2(silu(layer.w1(h2)) * layer.w3(h2))
        return x

    def head0(self, x_last: np.ndarray):
        """Final slow norm, tied codebook-0 head: returns (logits [V0], h_t [d])."""
        h = rmsnorm(x_last, self.slow_final_norm, self.dims.rms_eps)
        return h @ self.w0.T, h

    def fast_logits(self, y: np.ndarray):
        z = rmsnorm(y, self.fast_final_norm, self.dims.rms_eps)
        return self.fast_head(z)


class OracleDecoder:
    """Batch-1 decode state: slow KV cache, position, committed frames.

    Greedy by default. With `sampling` (oracle/sampling.SamplingParams) and
    `uniforms` ([max_len][1 + n_res] values in [0, 1)), the code of codebook k
    of the frame at slow position p is drawn by sample_code with uniforms[p][k],
    its repetition window reading the committed codes of the frames since the
    prompt (the first frame sits at the last prompt position)."""

    def __init__(self, model: OracleModel, max_len: int, sampling=None, uniforms=None):
        d = model.dims
        self.m = model
        self.max_len = max_len
        shape = (d.n_layers_slow, max_len, d.n_heads_kv, d.head_dim)
        self.k = np.zeros(shape, dtype=model.dt)
        self.v = np.zeros(shape, dtype=model.dt)
        self.pos = 0
        self.last_c0 = None
        self.sampling = sampling
        self.uniforms = uniforms
        self.ring = np.full((max_len, d.n_res + 1), -1, dtype=np.int64)
        self.first = 0          # slow position of frame 0
        self.frame_pos = 0      # slow position of the frame being produced
        self.margins = []       # sample_code's info per sampled code, in order

    def _choose(self, logits, k):
        """The model's code for codebook k of the current frame."""
        if self.sampling is None:
            return greedy_argmax(logits)
        from .sampling import sample_code, window_history
        p = self.frame_pos
        hist = window_history(self.ring, p, k, self.first, self.sampling.window)
        code, info = sample_code(logits, hist, self.sampling, float(self.uniforms[p][k]))
        self.margins.append(info)
        return code

    def _slow(self, x: np.ndarray, p0: int):
        for i, layer in enumerate(self.m.slow):
            x = self.m.block(layer, x, p0, self.k[i], self.v[i])
        return x

    def fast_frame(self, h_t: np.ndarray, c0: int, forced=None):
        """Fast AR over one frame. Returns (codes [R], logits [R][Vr]) for codebooks 1..R."""
        m, d = self.m, self.m.dims
        R = d.n_res
        fk = np.zeros((d.n_layers_fast, R + 1, d.n_heads_kv, d.head_dim), dtype=m.dt)
        fv = np.zeros_like(fk)

        def run(u, p):
            y = u[None, :]
            for i, layer in enumerate(m.fast):
                y = m.block(layer, y, p, fk[i], fv[i])
            return y[0]

        run(h_t, 0)                                    # fast position 0: output unused
        prev = c0 if forced is None else int(forced[0])
        codes, logits = [], []
        for k in range(1, R + 1):
            y = run(m.fast_emb[k - 1][prev], k)
            lk = m.fast_logits(y)
            ck = self._choose(lk, k)
            codes.append(ck)
            logits.append(lk)
            prev = ck if forced is None else int(forced[k])
            self.ring[self.frame_pos][k] = prev
        return codes, logits

    def _frame_from_slow(self, x_last, forced):
        l0, h_t = self.m.head0(x_last)
        c0 = self._choose(l0, 0)
        codes, logits = [c0], [l0]
        committed_c0 = c0 if forced is None else int(forced[0])
        self.ring[self.frame_pos][0] = committed_c0
        if self.m.dims.has_fast:
            cs, ls = self.fast_frame(h_t, c0, forced)
            codes += cs
            logits += ls
        self.last_c0 = committed_c0
        return np.array(codes, dtype=np.int32), logits

    def prefill(self, tokens, forced=None, block: bool = True):
        """Prompt ids -> frame 0. block=True runs the prompt as one causal block,
        block=False as one slow step per token (the two are equal)."""
        tokens = np.asarray(tokens)
        n = len(tokens)
        if n < 1 or n > self.max_len:
            raise ValueError("prompt length")
        x = self.m.w0[tokens]
        if block:
            x = self._slow(x, 0)
            x_last = x[-1]
        else:
            for p in range(n):
                x_last = self._slow(x[p:p + 1], p)[0]
        self.pos = n
        self.first = self.frame_pos = n - 1
        return self._frame_from_slow(x_last, forced)

    def decode_frame(self, forced=None):
        """One frame: slow step on the previous committed c0 at position pos, then the fast AR."""
        if self.last_c0 is None:
            raise RuntimeError("decode before prefill")
        if self.pos >= self.max_len:
            raise RuntimeError("capacity")
        x = self.m.w0[self.last_c0][None, :]
        x = self._slow(x, self.pos)[0]
        self.frame_pos = self.pos
        self.pos += 1
        return self._frame_from_slow(x, forced)


def full_recompute_slow(model: OracleModel, tokens):
    """Cache-free causal pass over a whole slow input sequence.

    Attention is formed as multi-head attention with each KV head repeated
    n_q / n_kv times. Returns (logits0 [n][V0], h_t [n][d]).
    """
    d = model.dims
    tokens = np.asarray(tokens)
    x = model.w0[tokens]
    return _full(model, model.slow, x, d, final=lambda y: model.head0(y))


def full_recompute_fast(model: OracleModel, h_t, codes_in):
    """Cache-free causal pass over [h_t, E0[c0], ..., E_{R-1}[c_{R-1}]]; logits at positions 1..R."""
    d = model.dims
    rows = [h_t] + [model.fast_emb[k][int(codes_in[k])] for k in range(d.n_res)]
    x = np.stack(rows).astype(model.dt)
    logits = _full(model, model.fast, x, d, final=lambda y: (model.fast_logits(y), None))[0]
    return logits[1:]


def _full(model, layers, x, d, final):
    n = x.shape[0]
    hd = d.head_dim
    g = d.group
    cos, sin = rope_cos_sin(np.arange(n), hd, d.rope_base, model.dt)
    causal = np.tril(np.ones((n, n), dtype=bool))
    scale = model.dt(1.0 / np.sqrt(hd))
    for layer in layers:
        h = rmsnorm(x, layer.attn_norm, d.rms_eps)
        qkv = layer.wqkv(h)
        q = qkv[:, :d.q_width].reshape(n, d.n_heads_q, hd)
        k = qkv[:, d.q_width:d.q_width + d.kv_width].reshape(n, d.n_heads_kv, hd)
        v = qkv[:, d.q_width + d.kv_width:].reshape(n, d.n_heads_kv, hd)
        q = apply_rope(q, cos[:, None, :], sin[:, None, :])
        k = apply_rope(k, cos[:, None, :], sin[:, None, :])
        if model.kv_bf16:
            k, v = round_bf16(k), round_bf16(v)
        k_rep = np.repeat(k, g, axis=1)                               # [n, n_q, hd]
        v_rep = np.repeat(v, g, axis=1)
        s = np.einsum("ihd,jhd->hij", q, k_rep) * scale               # [n_q, n, n]
        s = np.where(causal[None], s, -np.inf)
        s = s - s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=2, keepdims=True)
        o = np.einsum("hij,jhd->ihd", p, v_rep).reshape(n, d.q_width)
        x = x + layer.wo(o)
        h2 = rmsnorm(x, layer.ffn_norm, d.rms_eps)
        x = x + layer.w2(silu(layer.w1(h2)) * layer.w3(h2))
    return final(x)
