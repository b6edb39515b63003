"""Model shapes and run recipes for the Dual-AR (RQ-Transformer) decode frame.

Shapes follow the Fish-Speech S2-Pro geometry described on the pages:
  * tuna-fish README, "Inference estimation": slow AR 36 layers and fast AR 4
    layers, KV width C_kv = 1024, max_length 1024, batch 1;
  * tuna-fish README, "Inference speedtest": the run recipe prefill 128 then
    decode 896 to a 1024-long context;
  * groxaxo fork README, architecture paragraph, and the s2-pro-fp8 model card,
    "Architecture": ten codebooks per frame, i.e. codebook 0 from the slow AR
    plus nine residual codebooks from the fast AR;
  * pyshine fish-speech tour, "Why You Need This": rotary embeddings and
    grouped-query attention in a decoder-only transformer.
Widths (d 2560, 32/8 heads of 128, SwiGLU 9728, 4096-entry codebooks) are the
workload's own; the tiny shape exists so a CPU oracle finishes in seconds.

The canonical tensor list below fixes (a) names, (b) shapes, (c) the order in
which tensors are drawn from the seed. All matrices are row-major [out][in].
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DarDims:
    """Geometry of one Dual-AR model."""

    name: str
    n_layers_slow: int
    n_layers_fast: int
    d_model: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    ffn_dim: int
    vocab_c0: int      # codebook-0 entries (slow head / tied input table)
    vocab_res: int     # entries of each residual codebook
    n_res: int         # residual codebooks emitted by the fast AR per frame
    rms_eps: float = 1e-6
    rope_base: float = 1e6

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads_q + 2 * self.n_heads_kv) * self.head_dim

    @property
    def q_width(self) -> int:
        return self.n_heads_q * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_heads_kv * self.head_dim

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def frame_codes(self) -> int:
        return 1 + self.n_res

    @property
    def has_fast(self) -> bool:
        return self.n_res > 0 and self.n_layers_fast > 0


@dataclass(frozen=True)
class Workload:
    """A run: a model, a weight precision, a batch, prompt and decode lengths."""

    name: str
    dims: DarDims
    wtype: str              # "bf16", "fp8", "int8" or "int4"
    batch: int
    prefill_len: int        # per sequence (batch 1) or the minimum (ragged)
    prefill_len_max: int    # == prefill_len unless ragged
    decode_frames: int
    max_len: int
    weight_seed: int = 0
    prompt_seed: int = 1
    length_seed: int = 2
    # continuous batching (requests > 0): `batch` slots serve `requests`
    # requests, prompts prefill_len..prefill_len_max ids, each decoding
    # frames_min..decode_frames frames; slow KV in pages of page_len positions
    requests: int = 0
    frames_min: int = 0
    page_len: int = 0
    n_pages: int = 0


TINY = DarDims(
    name="tiny", n_layers_slow=2, n_layers_fast=1, d_model=256, n_heads_q=4,
    n_heads_kv=2, head_dim=64, ffn_dim=768, vocab_c0=1024, vocab_res=256, n_res=3,
)
S2_SLOW_ONLY = DarDims(
    name="s2pro_slow", n_layers_slow=36, n_layers_fast=0, d_model=2560, n_heads_q=32,
    n_heads_kv=8, head_dim=128, ffn_dim=9728, vocab_c0=4096, vocab_res=0, n_res=0,
)
S2_DUAL = replace(S2_SLOW_ONLY, name="s2pro_dual", n_layers_fast=4, vocab_res=4096, n_res=9)

DIMS = {"tiny": TINY, "s2pro_slow": S2_SLOW_ONLY, "s2pro_dual": S2_DUAL}

WORKLOADS = {
    # tiny Dual-AR; the oracle runs it in full (prefill 16, 16 frames)
    "tiny_bf16": Workload("tiny_bf16", TINY, "bf16", 1, 16, 16, 16, 32),
    "tiny_fp8": Workload("tiny_fp8", TINY, "fp8", 1, 16, 16, 16, 32),
    "tiny_int8": Workload("tiny_int8", TINY, "int8", 1, 16, 16, 16, 32),
    "tiny_int4": Workload("tiny_int4", TINY, "int4", 1, 16, 16, 16, 32),
    # slow AR only, full shape: prefill 128 then 896 tokens to length 1024
    "s2pro_slow_bf16": Workload("s2pro_slow_bf16", S2_SLOW_ONLY, "bf16", 1, 128, 128, 896, 1024),
    # full Dual-AR frame, full shape, bf16 and per-row fp8
    "s2pro_dual_bf16": Workload("s2pro_dual_bf16", S2_DUAL, "bf16", 1, 128, 128, 896, 1024),
    "s2pro_dual_fp8": Workload("s2pro_dual_fp8", S2_DUAL, "fp8", 1, 128, 128, 896, 1024),
    # the same frame with per-row int8 weight-only matrices (the tuna-fish README's int8wo mode)
    "s2pro_dual_int8": Workload("s2pro_dual_int8", S2_DUAL, "int8", 1, 128, 128, 896, 1024),
    # and with int4 weight-only matrices, a scale per 128 columns (its int4wo mode)
    "s2pro_dual_int4": Workload("s2pro_dual_int4", S2_DUAL, "int4", 1, 128, 128, 896, 1024),
    # batched Dual-AR decode, ragged prompts 128..512, max length 4096
    "s2pro_dual_b16": Workload("s2pro_dual_b16", S2_DUAL, "bf16", 16, 128, 512, 3584, 4096),
    "s2pro_dual_b64": Workload("s2pro_dual_b64", S2_DUAL, "bf16", 64, 128, 512, 3584, 4096),
    # continuous batching: 16 slots serve 64 requests (prompts 128..512, 64..1024
    # frames each), slow KV from a pool of 256-position pages sized for 16 of
    # the longest requests (6 pages each) plus the parking page
    "s2pro_dual_cb16": Workload("s2pro_dual_cb16", S2_DUAL, "bf16", 16, 128, 512, 1024, 4096,
                                requests=64, frames_min=64, page_len=256, n_pages=97),
    # and 64 slots serving 256 requests from a pool sized the same way (6 pages per slot)
    "s2pro_dual_cb64": Workload("s2pro_dual_cb64", S2_DUAL, "bf16", 64, 128, 512, 1024, 4096,
                                requests=256, frames_min=64, page_len=256, n_pages=385),
}


def tensor_specs(dims: DarDims):
    """Canonical tensor list: (name, shape, kind) with kind in {emb, norm, linear}.

    Slow AR: a tied table w0 [V0][d] that is both the codebook-0 head and the
    input table of the slow AR, then per layer the pre-norm LLaMA block
    (attn_norm, fused wqkv, wo, ffn_norm, w1, w3, w2), then a final norm.
    Fast AR: one input table per codebook it consumes (codebook k feeds the
    fast step that predicts codebook k+1), the same block per layer, a final
    norm and one output head shared by all residual codebooks.
    """
    d, F = dims.d_model, dims.ffn_dim
    specs = [("w0", (dims.vocab_c0, d), "emb")]

    def block(prefix):
        return [
            (f"{prefix}.attn_norm", (d,), "norm"),
            (f"{prefix}.wqkv", (dims.qkv_rows, d), "linear"),
            (f"{prefix}.wo", (d, dims.q_width), "linear"),
            (f"{prefix}.ffn_norm", (d,), "norm"),
            (f"{prefix}.w1", (F, d), "linear"),
            (f"{prefix}.w3", (F, d), "linear"),
            (f"{prefix}.w2", (d, F), "linear"),
        ]

    for layer in range(dims.n_layers_slow):
        specs += block(f"slow.{layer}")
    specs.append(("slow.final_norm", (d,), "norm"))
    if dims.has_fast:
        for k in range(dims.n_res):
            rows = dims.vocab_c0 if k == 0 else dims.vocab_res
            specs.append((f"fast.emb.{k}", (rows, d), "emb"))
        for layer in range(dims.n_layers_fast):
            specs += block(f"fast.{layer}")
        specs.append(("fast.final_norm", (d,), "norm"))
        specs.append(("fast.head", (dims.vocab_res, d), "linear"))
    return specs


def linear_names(dims: DarDims):
    """Names of the nn.Linear-style matrices (the ones per-row fp8 quantises)."""
    return [name for name, _, kind in tensor_specs(dims) if kind == "linear"]
