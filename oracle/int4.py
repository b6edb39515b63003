"""Group-wise symmetric int4 weight-only quantiser (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The tuna-fish README times torchao's int4 weight-only mode ("int4wo", its
fastest mode) next to fp8 and int8; the pages give neither a formula nor a
group size. The reading taken: each output row is cut into groups of 128
consecutive input columns (128 divides every width of the model); a group gets
its own fp32 scale s = max |w| / 7 over the group, q = round-half-to-even(w / s)
with an fp32 division, clamped to [-7, 7]; a zero group has s = 0 and codes 0.
Dequantisation is s * q. Storage: two codes per byte, column 2j in the low
nibble and column 2j + 1 in the high nibble, two's complement.
"""
from __future__ import annotations

import numpy as np

INT4_MAX = 7
GROUP = 128


def quantize_int4_groups(w: np.ndarray):
    """[rows][cols] fp32 -> (codes int8 [rows][cols] in [-7, 7], scale fp32 [rows][cols / 128])."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 128")
    g = w.reshape(rows, cols // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    scale = (amax / np.float32(INT4_MAX)).astype(np.float32)
    codes = np.zeros(g.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        ratio = (g[nz] / scale[nz][:, None]).astype(np.float32)
        codes[nz] = np.clip(np.rint(ratio), -INT4_MAX, INT4_MAX).astype(np.int8)
    return codes.reshape(rows, cols), scale


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes [rows][cols] (cols even) -> uint8 [rows][cols / 2], even column in the low nibble."""
    c = np.asarray(codes, dtype=np.int8).astype(np.uint8) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows][cols / 2] -> int8 codes [rows][cols] (sign-extended nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo).astype(np.int8)
    hi = np.where(hi > 7, hi - 16, hi).astype(np.int8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequantize_int4(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """s_g * q in fp64, [rows][cols]."""
    rows, cols = codes.shape
    return (codes.astype(np.float64).reshape(rows, cols // GROUP, GROUP) *
            scale.astype(np.float64)[:, :, None]).reshape(rows, cols)
