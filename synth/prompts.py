"""Seeded prompt token ids, sampling draws and logit rows for the sampler.

The pages drive decode with a text+audio prompt that is not available here;
uniform random ids over the codebook-0 table stand in for it, with the pages'
prompt lengths (tuna-fish README, "Inference speedtest": prefill 128).
"""
from __future__ import annotations

import numpy as np


def gen_prompt(n: int, vocab: int, seed: int = 1) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def gen_ragged_prompts(batch: int, lo: int, hi: int, vocab: int, seed: int = 1, length_seed: int = 2):
    """Independent prompts with lengths uniform on [lo, hi] (inclusive)."""
    lrng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([length_seed])))
    lens = lrng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    prompts = []
    for b in range(batch):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
        prompts.append(rng.integers(0, vocab, size=int(lens[b]), dtype=np.int64).astype(np.int32))
    return lens, prompts


def gen_requests(n: int, lo: int, hi: int, frames_lo: int, frames_hi: int, vocab: int, seed: int = 1,
                 length_seed: int = 2):
    """A stream of n requests: prompt lengths uniform on [lo, hi], frame
    counts uniform on [frames_lo, frames_hi] (inclusive), random prompt ids."""
    lens, prompts = gen_ragged_prompts(n, lo, hi, vocab, seed, length_seed)
    frng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([length_seed, 1])))
    frames = frng.integers(frames_lo, frames_hi + 1, size=n, dtype=np.int64).astype(np.int32)
    return lens, frames, prompts


def gen_uniforms(max_len: int, batch: int, codes: int, seed: int = 3) -> np.ndarray:
    """Draws for sampling: fp32 [max_len][batch][codes], uniform on [0, 1)."""
    rng = np.random.default_rng(seed)
    return rng.random((max_len, batch, codes), dtype=np.float32)


def gen_sample_logits(rows: int, V: int, seed: int, scale: float = 3.0, ties: bool = False) -> np.ndarray:
    """fp32 [rows][V] logit rows for the sampling step: normal * scale; with
    ties, every row repeats a few of its values (equal candidates)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, V)) * scale).astype(np.float32)
    if ties:
        for r in range(rows):
            src = rng.integers(0, V, 8)
            dst = rng.integers(0, V, 8)
            x[r, dst] = x[r, src]
    return x
