"""Shapes, seeded weights and codes for the RVQ codec decoder (codes -> waveform).

What the pages fix (tuna-fish README, intro and "Audio tokenizer speedtest";
pyshine fish-speech tour, "Why You Need This"): a modified DAC-style
convolutional codec, a residual vector quantiser of ten stacked codebooks, a
latent rate of roughly 21 Hz, and 44.1 kHz mono audio (the speedtest feeds
[1, 1, 340982] samples for a 7.73 s clip). 44100 / 2048 = 21.5 Hz, so one latent
frame becomes 2048 samples. The codebooks share the Dual-AR model's vocabulary
(4096 entries each).

What they leave open is taken from the published DAC decoder design for
44.1 kHz audio: a 7-tap input convolution from the latent width 1024 to 1536
channels, upsampling blocks that each halve the width (Snake, transposed
convolution with kernel 2*stride, three residual units with dilations 1, 3, 9),
then Snake, a 7-tap convolution to one channel and tanh. Only the strides change,
(8, 8, 8, 4) instead of (8, 8, 4, 2), so that the blocks upsample 2048-fold.

No arithmetic of the method lives here: only names, shapes and random draws.
Every tensor is drawn from PCG64(SeedSequence([seed, 7, index])) in the order of
codec_tensor_specs and rounded to bf16 (nearest even); the bf16 bit tensor is
the canonical weight both the oracle and the GPU consume.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .weights import f32_to_bf16_bits


@dataclass(frozen=True)
class CodecDims:
    name: str
    n_codebooks: int
    codebook_size: int
    latent_dim: int
    channels: int              # width after the input convolution; halves in every block
    rates: tuple               # upsampling stride of each block (even)
    dilations: tuple = (1, 3, 9)
    kernel: int = 7            # taps of the input, residual and output convolutions
    sample_rate: int = 44100

    @property
    def hop(self) -> int:
        return int(np.prod(self.rates))

    @property
    def widths(self):
        """Channel count at the input of each block, then after the last block."""
        return [self.channels >> i for i in range(len(self.rates) + 1)]


S2_CODEC = CodecDims("s2pro_codec", n_codebooks=10, codebook_size=4096, latent_dim=1024, channels=1536,
                     rates=(8, 8, 8, 4))
# tiny shape: the oracle finishes in well under a second; widths 128 -> 64 -> 32
TINY_CODEC = CodecDims("tiny_codec", n_codebooks=10, codebook_size=64, latent_dim=64, channels=128, rates=(2, 4))

# a second small shape for the layer forms the first does not reach: 5-tap
# convolutions, two residual units per block (dilations 1, 2), three blocks,
# and a 256-channel block whose units take the two-launch path; widths
# 256 -> 128 -> 64 -> 32
SMALL_CODEC_K5 = CodecDims("small_codec_k5", n_codebooks=4, codebook_size=32, latent_dim=96, channels=256,
                           rates=(2, 2, 4), dilations=(1, 2), kernel=5)

CODEC_DIMS = {"s2pro_codec": S2_CODEC, "tiny_codec": TINY_CODEC, "small_codec_k5": SMALL_CODEC_K5}


@dataclass(frozen=True)
class CodecWorkload:
    name: str
    dims: CodecDims
    frames: int                # latent frames decoded (audio = frames * hop samples)
    weight_seed: int = 0
    code_seed: int = 3


CODEC_WORKLOADS = {
    # 37 frames: several 128-row tiles of every layer plus ragged tails
    "tiny_codec": CodecWorkload("tiny_codec", TINY_CODEC, 37),
    # the speedtest's 7.73 s clip ([1, 1, 340982] samples) padded to whole hops: 167 frames
    "s2pro_codec_7s": CodecWorkload("s2pro_codec_7s", S2_CODEC, math.ceil(340982 / 2048)),
    # its 27.70 s clip ([1, 1, 1221570] samples): 597 frames
    "s2pro_codec_28s": CodecWorkload("s2pro_codec_28s", S2_CODEC, math.ceil(1221570 / 2048)),
}

# standard deviations of the draws: tables N(0, 0.1^2) (ten of them summed);
# convolution weights N(0, (gain / sqrt(fan_in))^2) with fan_in the inputs that
# reach one output (Cin * taps, Cin * 2 for a transposed convolution with kernel
# 2*stride); the second convolution of a residual unit has gain 0.3 so the
# residual stream grows slowly, and the output convolution gain 0.3 so the
# samples before tanh have a standard deviation near 0.5 (tanh mostly
# unsaturated); biases N(0, 0.02^2); Snake alphas uniform on [0.5, 1.5)
TABLE_STD = 0.1
BIAS_STD = 0.02
RES_GAIN = 0.3
OUT_GAIN = 0.3


def codec_tensor_specs(d: CodecDims):
    """Canonical tensor list: (name, shape, kind, std). PyTorch layouts:
    convolution weights [Cout][Cin][taps], transposed convolution [Cin][Cout][taps]."""
    K = d.kernel
    w = d.widths
    specs = [(f"codec.rvq.{k}", (d.codebook_size, d.latent_dim), "normal", TABLE_STD) for k in range(d.n_codebooks)]
    specs += [("codec.in.w", (w[0], d.latent_dim, K), "normal", 1.0 / math.sqrt(d.latent_dim * K)),
              ("codec.in.b", (w[0],), "normal", BIAS_STD)]
    for i, s in enumerate(d.rates):
        cin, cout = w[i], w[i + 1]
        p = f"codec.b{i}"
        specs += [(f"{p}.alpha", (cin,), "alpha", 0.0),
                  (f"{p}.up.w", (cin, cout, 2 * s), "normal", 1.0 / math.sqrt(cin * 2)),
                  (f"{p}.up.b", (cout,), "normal", BIAS_STD)]
        for j in range(len(d.dilations)):
            r = f"{p}.ru{j}"
            specs += [(f"{r}.alpha1", (cout,), "alpha", 0.0),
                      (f"{r}.w1", (cout, cout, K), "normal", 1.0 / math.sqrt(cout * K)),
                      (f"{r}.b1", (cout,), "normal", BIAS_STD),
                      (f"{r}.alpha2", (cout,), "alpha", 0.0),
                      (f"{r}.w2", (cout, cout, 1), "normal", RES_GAIN / math.sqrt(cout)),
                      (f"{r}.b2", (cout,), "normal", BIAS_STD)]
    specs += [("codec.out.alpha", (w[-1],), "alpha", 0.0),
              ("codec.out.w", (1, w[-1], K), "normal", OUT_GAIN / math.sqrt(w[-1] * K)),
              ("codec.out.b", (1,), "normal", BIAS_STD)]
    return specs


def _draw(index, shape, kind, std, seed):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7, index])))
    if kind == "alpha":
        x = rng.uniform(0.5, 1.5, size=shape).astype(np.float32)
    else:
        x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(x)


def gen_codec_weights(d: CodecDims, seed: int = 0):
    """{name: uint16 array of bf16 bits} for every codec tensor."""
    return {name: _draw(i, shape, kind, std, seed) for i, (name, shape, kind, std) in enumerate(codec_tensor_specs(d))}


def gen_codes(frames: int, d: CodecDims, seed: int = 3) -> np.ndarray:
    """Random codes, frame-major int32 [frames][n_codebooks] (the Dual-AR model's
    frame layout), uniform over each codebook."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    return rng.integers(0, d.codebook_size, size=(frames, d.n_codebooks), dtype=np.int64).astype(np.int32)
