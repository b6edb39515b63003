"""Seeded random-init weights, stored as bfloat16 bit patterns (uint16).

Every tensor is drawn from its own stream, PCG64(SeedSequence([seed, index]))
where index is the tensor's position in the canonical list, so any subset can
be regenerated without drawing the rest. Linear and embedding entries are
N(0, 0.02^2); norm gains are 1 + N(0, 0.02^2) (a gain drawn around zero would
shrink every normalised vector fifty-fold with random signs and flatten the
logits). The fp32 draw is rounded to bf16 with round-to-nearest-even; the bf16
bit tensor is the canonical weight that both the oracle and the GPU consume.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import DarDims, tensor_specs

STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def gen_tensor(dims: DarDims, name: str, seed: int = 0) -> np.ndarray:
    """Regenerate one canonical tensor (uint16 bf16 bits) by name."""
    specs = tensor_specs(dims)
    for index, (n, shape, kind) in enumerate(specs):
        if n == name:
            return _draw(index, shape, kind, seed)
    raise KeyError(name)


def _draw(index, shape, kind, seed):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(STD)
    if kind == "norm":
        x += np.float32(1.0)
    return f32_to_bf16_bits(x)


def gen_weights(dims: DarDims, seed: int = 0, names=None, threads: int | None = None):
    """All (or the named) canonical tensors as {name: uint16 array of bf16 bits}."""
    specs = tensor_specs(dims)
    wanted = [(i, s) for i, s in enumerate(specs) if names is None or s[0] in names]
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    out = {}

    def work(item):
        index, (name, shape, kind) = item
        return name, _draw(index, shape, kind, seed)

    if threads <= 1 or len(wanted) <= 1:
        for item in wanted:
            name, t = work(item)
            out[name] = t
    else:
        with ThreadPoolExecutor(threads) as pool:
            for name, t in pool.map(work, wanted):
                out[name] = t
    return out
