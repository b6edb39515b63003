"""Per-row symmetric int8 weight-only quantiser (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The tuna-fish README lists torchao's int8 weight-only mode ("int8wo") among its
quantised decode modes and times it ("Inference estimation" and its
throughput table); the pages give no formula for it. The reading taken is the
plainest symmetric per-output-channel scheme, the same shape as the fp8 card's
per-row scheme: every output row gets its own fp32 scale s = max_j |w_j| / 127,
q_j = round-half-to-even(w_j / s) with an fp32 division, clamped to
[-127, 127]; a zero row has s = 0 and codes 0. Dequantisation is s * q.
"""
from __future__ import annotations

import numpy as np

INT8_MAX = 127


def quantize_int8_rows(w: np.ndarray):
    """Per-row symmetric int8 quantisation of a [rows][cols] fp32 matrix.

    Returns (codes int8 [rows][cols], scale fp32 [rows]).
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    scale = (amax / np.float32(INT8_MAX)).astype(np.float32)
    codes = np.zeros(w.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        ratio = (w[nz] / scale[nz][:, None]).astype(np.float32)
        codes[nz] = np.clip(np.rint(ratio), -INT8_MAX, INT8_MAX).astype(np.int8)
    return codes, scale
