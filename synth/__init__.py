"""Seeded synthetic inputs for the Dual-AR decode frame: model shapes, weights, prompts.

This package holds no arithmetic of the method itself. It only fixes shapes and
draws random numbers, so that the CPU oracle, the tests and the benchmark all
see the same bytes. The quantiser, the norms, the attention and everything else
the method computes live elsewhere (the oracle has its own copy, the HIP library
has its own).
"""
from .configs import (  # noqa: F401
    DarDims,
    Workload,
    DIMS,
    WORKLOADS,
    tensor_specs,
    linear_names,
)
from .weights import gen_weights, gen_tensor, f32_to_bf16_bits  # noqa: F401
from .prompts import gen_prompt, gen_ragged_prompts, gen_requests, gen_sample_logits, gen_uniforms  # noqa: F401
from .codec import (  # noqa: F401
    CodecDims,
    CodecWorkload,
    CODEC_DIMS,
    CODEC_WORKLOADS,
    codec_tensor_specs,
    gen_codec_weights,
    gen_codes,
)
