"""CPU oracle for the batch-1 Dual-AR (RQ-Transformer) decode frame.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, unfused definition
of what the decode path computes, in NumPy fp32 (fp64 where stated). Only the
tests, the package smoke check and the benchmark's CPU-baseline leg may import
it. It shares no code with the HIP library and never imports it; the HIP path
never imports this package.

Pinned against what the pages and the mathematics fix (see tests/test_oracle_*):
  fp8.py    e4m3fn decode/encode and the per-row symmetric quantiser
            (s2-pro-fp8 model card, "Quantization Details")
  model.py  RMSNorm, rotary embedding, GQA attention, the pre-norm SwiGLU block,
            the slow AR step, the fast AR frame loop, prefill, decode and a
            cache-free full recompute (tuna-fish README, intro and "Inference
            estimation"; groxaxo fork README, architecture paragraph; pyshine
            fish-speech tour, "Why You Need This")
  int8.py, int4.py  weight-only quantisers (tuna-fish README's int8wo and
            int4wo modes; readings in their headers)
  sampling.py  temperature / top-k / top-p / repetition-window sampling of
            one code (pyshine fish-speech tour, "Why You Need This"; reading
            in its header)
  codec.py  RVQ decode and the DAC-style convolutional decoder, codes to
            waveform (tuna-fish README, intro and "Audio tokenizer speedtest";
            pyshine fish-speech tour, "Why You Need This"; readings in its header)
End-to-end logits have no printed values on the pages: parity unpinned at that
level; the pins are the parts and the invariants that tie them together.
"""
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode_table,
    e4m3_decode,
    e4m3_encode,
    quantize_rows,
)
from .model import (  # noqa: F401
    bf16_to_f32,
    round_bf16,
    rmsnorm,
    silu,
    rope_cos_sin,
    apply_rope,
    gqa_attention,
    Linear,
    OracleModel,
    OracleDecoder,
    greedy_argmax,
    full_recompute_slow,
    full_recompute_fast,
)
from .codec import (  # noqa: F401
    rvq_decode,
    snake,
    conv1d,
    conv_transpose1d,
    CodecParams,
    codec_decode,
    receptive_halo,
)
