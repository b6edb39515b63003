"""RVQ codec decode, codes -> waveform, written out plainly (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, and where the pages say so:
  * The codec is a modified DAC: a convolutional encoder-decoder with a
    residual vector quantiser of ten stacked codebooks at roughly 21 Hz; the
    first codebook holds the coarsest shape and each further one quantises the
    residual the previous ones left (pyshine fish-speech tour, "Why You Need
    This"; tuna-fish README, intro: "DAC style RVQ Audio Codec"). Decoding the
    quantiser therefore sums the ten selected codebook vectors of a frame.
  * The decoder upsamples the latent frames to 44.1 kHz audio (tuna-fish
    README, "Audio tokenizer speedtest": [1, 1, 340982] samples for 7.73 s).

Readings where the pages leave a step open (each also listed in the design doc):
  * z[t] = sum_k table_k[code[t][k]] with the tables in the latent width (no
    low-dimensional factorised lookup).
  * Decoder layers as in the published DAC decoder: a 7-tap convolution to
    the first width; per block Snake, a transposed convolution with kernel
    2*stride, stride `stride`, padding stride/2 (output length T * stride),
    and three residual units x + conv_1(Snake(conv_7,dil(Snake(x)))) with
    dilations 1, 3, 9 (zero "same" padding); finally Snake, a 7-tap
    convolution to one channel and tanh. Weight normalisation is folded into
    plain weights; every convolution has a bias.
  * Snake(x) = x + sin(alpha x)^2 / alpha with one alpha per channel.
  * Precision: fp64 throughout, or with act="bf16" every convolution's input
    rounded to bf16 (nearest even, from its fp32 value) while weights, sums,
    biases and the residual stream stay wide: the activation precision the
    GPU decoder runs at (the pages time the codec in fp32 and fp16).

Layouts: activations are time-major [T][C]; weights follow PyTorch,
convolution [Cout][Cin][taps] and transposed convolution [Cin][Cout][taps].
"""
from __future__ import annotations

import numpy as np

from .model import bf16_to_f32, round_bf16


def rvq_decode(codes: np.ndarray, tables) -> np.ndarray:
    """z[t] = sum over codebooks k of tables[k][codes[t][k]], summed in k order."""
    codes = np.asarray(codes)
    T, nq = codes.shape
    z = np.zeros((T, tables[0].shape[1]), dtype=np.float64)
    for k in range(nq):
        z += tables[k][codes[:, k]]
    return z


def snake(x: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """x + sin(alpha x)^2 / alpha, alpha per channel (last axis)."""
    return x + np.sin(alpha * x) ** 2 / alpha


def conv1d(x: np.ndarray, w: np.ndarray, b: np.ndarray, dilation: int = 1) -> np.ndarray:
    """Same-length convolution (cross-correlation, as in deep-learning layers):
    y[t][o] = b[o] + sum_j sum_c w[o][c][j] x[t + dilation (j - (K-1)/2)][c],
    x taken as zero outside [0, T). x [T][Cin], w [Cout][Cin][K] with K odd."""
    T = x.shape[0]
    K = w.shape[2]
    half = (K - 1) // 2
    y = np.tile(np.asarray(b, dtype=np.float64), (T, 1))
    for j in range(K):
        off = dilation * (j - half)
        lo, hi = max(0, -off), min(T, T - off)
        if lo < hi:
            y[lo:hi] += x[lo + off:hi + off] @ np.ascontiguousarray(w[:, :, j].T)
    return y


def conv_transpose1d(x: np.ndarray, w: np.ndarray, b: np.ndarray, stride: int) -> np.ndarray:
    """Transposed convolution, kernel K = 2 stride, padding stride/2: input
    sample i adds x[i] W[:, :, k] to output o = i stride - stride/2 + k, kept
    for 0 <= o < T stride. x [T][Cin], w [Cin][Cout][K]."""
    assert stride % 2 == 0 and w.shape[2] == 2 * stride
    T = x.shape[0]
    pad = stride // 2
    n_out = T * stride
    y = np.tile(np.asarray(b, dtype=np.float64), (n_out, 1))
    for k in range(w.shape[2]):
        o = np.arange(T) * stride - pad + k
        ok = (o >= 0) & (o < n_out)
        y[o[ok]] += x[ok] @ np.ascontiguousarray(w[:, :, k])
    return y


class CodecParams:
    """The canonical bf16 weights widened to fp64, by name."""

    def __init__(self, dims, host: dict):
        self.dims = dims
        self.p = {name: bf16_to_f32(bits).astype(np.float64) for name, bits in host.items()}

    def __getitem__(self, name):
        return self.p[name]


def codec_decode(codes: np.ndarray, P: CodecParams, act: str | None = None) -> np.ndarray:
    """Audio samples [T * hop] from frame-major codes [T][n_codebooks]."""
    d = P.dims
    q = (lambda a: round_bf16(a).astype(np.float64)) if act == "bf16" else (lambda a: a)
    z = rvq_decode(codes, [P[f"codec.rvq.{k}"] for k in range(d.n_codebooks)])
    x = conv1d(q(z), P["codec.in.w"], P["codec.in.b"])
    for i, s in enumerate(d.rates):
        p = f"codec.b{i}"
        x = conv_transpose1d(q(snake(x, P[f"{p}.alpha"])), P[f"{p}.up.w"], P[f"{p}.up.b"], s)
        for j, dil in enumerate(d.dilations):
            r = f"{p}.ru{j}"
            h = conv1d(q(snake(x, P[f"{r}.alpha1"])), P[f"{r}.w1"], P[f"{r}.b1"], dil)
            h = conv1d(q(snake(h, P[f"{r}.alpha2"])), P[f"{r}.w2"], P[f"{r}.b2"])
            x = x + h
    y = conv1d(q(snake(x, P["codec.out.alpha"])), P["codec.out.w"], P["codec.out.b"])
    return np.tanh(y[:, 0])


def receptive_halo(dims) -> int:
    """Latent frames on either side of frame t whose codes can change the
    samples of frame t (the decoder's receptive field in whole frames). Going
    back from the output: the last convolution reaches (K-1)/2 samples; in each
    block, from its output back to its input, the residual units reach
    dil (K-1)/2 samples each, and the transposed convolution maps a reach of r
    output samples to ceil(r / stride) + 1 input samples; the input
    convolution adds (K-1)/2 frames."""
    h = (dims.kernel - 1) // 2
    reach = h
    for s in reversed(dims.rates):
        reach += sum(dil * h for dil in dims.dilations)
        reach = -(-reach // s) + 1
    return reach + h
