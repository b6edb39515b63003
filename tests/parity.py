"""Shared GPU-vs-oracle comparison for decode runs (no arithmetic of the method).

The bar for floating point: per (frame, codebook) logit vector the relative L2
error ||l_gpu - l_oracle|| / ||l_oracle|| (max over vectors) stays within the
tolerance of the weight type (2e-2 bf16, 5e-2 fp8, 2e-2 int8 and int4: the
integer codes are exact in fp32 and bf16 like bf16 weights, and both sides
apply the same row or group scales, so the bf16 bar applies); argmax agreement over all
(frame, codebook) comparisons is at least 99 %; and where the oracle's top-1
minus top-2 margin exceeds 1e-2 the codes are identical.
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 2e-2, "fp8": 5e-2, "int8": 2e-2, "int4": 2e-2}


def margin(logits):
    s = np.sort(logits)
    return float(s[-1] - s[-2])


def compare_frames(gpu_frames, oracle_frames, dims, wtype):
    """gpu_frames/oracle_frames: lists of (codes [1+R], logits list/array per codebook)."""
    rels, agree, total, exact_fail = [], 0, 0, []
    for f, ((gc, gl), (oc, ol)) in enumerate(zip(gpu_frames, oracle_frames)):
        for k in range(dims.n_res + 1):
            V = dims.vocab_c0 if k == 0 else dims.vocab_res
            g = np.asarray(gl[k][:V], dtype=np.float64)
            o = np.asarray(ol[k][:V], dtype=np.float64)
            rels.append(np.linalg.norm(g - o) / np.linalg.norm(o))
            total += 1
            agree += int(gc[k] == oc[k])
            if margin(o) > 1e-2 and gc[k] != oc[k]:
                exact_fail.append((f, k, int(gc[k]), int(oc[k]), margin(o)))
    return {
        "max_rel": float(np.max(rels)),
        "median_rel": float(np.median(rels)),
        "agree": agree / total,
        "n": total,
        "exact_fail": exact_fail,
        "tol": TOL[wtype],
    }


def assert_parity(stats):
    assert stats["max_rel"] <= stats["tol"], stats
    assert stats["agree"] >= 0.99, stats
    assert not stats["exact_fail"], stats
