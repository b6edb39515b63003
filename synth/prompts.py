"""Seeded prompt token ids.

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
