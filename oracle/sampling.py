"""Sampling of one code from a codebook's logits (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pyshine fish-speech tour ("Why You Need This") says the generation loop
samples with top-p and top-k and keeps repetition windows; the pages give no
formula, order or defaults. The reading taken, the common one of LLM
generation loops, step by step for one codebook of one frame:

1. repetition window: every distinct code of this codebook among the
   previous `window` frames of the sequence (frames generated since its
   prompt; their committed codes) has its logit divided by `penalty` when
   positive and multiplied by it otherwise;
2. temperature: every logit divided by `temperature`;
3. top-k: the `top_k` largest values are the candidates (equal values: the
   lower code first);
4. softmax over the candidates, in the candidates' order (largest first);
5. top-p: the candidates are cut after the first one at which the running
   sum of probabilities reaches `top_p` times their total;
6. draw: with a uniform u in [0, 1) given from outside, the code is the first
   kept candidate whose running sum exceeds u times the kept total.

Arithmetic in fp32 like the kernel (the decisions then fall the same way
except at ties within fp32 rounding): fp32 division for the penalty and the
temperature, fp32 exp and sequential fp32 running sums. Besides the code,
`sample_code` reports how far the decisions were from flipping, so that a
comparison can skip draws that sit on a boundary.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class SamplingParams:
    temperature: float = 1.0
    top_k: int = 50
    top_p: float = 1.0
    penalty: float = 1.0
    window: int = 0


def penalise(logits, history, penalty):
    """Step 1: logits (fp32 copy) with the codes in `history` penalised once each."""
    v = np.array(logits, dtype=np.float32, copy=True)
    p = np.float32(penalty)
    for c in sorted({int(c) for c in history if 0 <= int(c) < v.size}):
        v[c] = v[c] / p if v[c] > 0 else v[c] * p
    return v


def sample_code(logits, history, params: SamplingParams, u: float):
    """Steps 1-6 for one logit vector. Returns (code, info) where info holds
    the kept candidates in order, their fp32 probabilities and running sums,
    and the margins: `logit_gap` between the last candidate and the first
    value left out (inf when all are kept), `mass_gap` the smallest relative
    distance of the top-p and draw thresholds from a running sum, `order_gap`
    between the picked candidate's value and its neighbours' in the order."""
    v = penalise(logits, history, params.penalty)
    v = v / np.float32(params.temperature)
    v = np.where(np.isnan(v), np.float32(-np.inf), v).astype(np.float32)
    V = v.size
    k = min(int(params.top_k), V)
    # descending value, ties by ascending code
    order = np.lexsort((np.arange(V), -v.astype(np.float64)))
    cand = order[:k]
    vals = v[cand]
    logit_gap = float(vals[-1]) - float(v[order[k]]) if k < V else np.inf
    w = np.exp((vals - vals[0]).astype(np.float32)).astype(np.float32)
    cum = np.cumsum(w, dtype=np.float32)
    total = cum[-1]
    thr = np.float32(params.top_p) * total
    m = int(np.argmax(cum >= thr)) + 1 if np.any(cum >= thr) else k
    S = cum[m - 1]
    target = np.float32(u) * S
    pick = int(np.sum(cum[:m] <= target))
    pick = min(pick, m - 1)
    # the cut moves if the running sum at it drops below the threshold (only
    # possible before the last candidate: at the last one the threshold is
    # at most the total) or the one before it reaches the threshold
    gaps = [abs(float(cum[m - 1]) - float(thr))] if m < k else []
    if m >= 2:
        gaps.append(abs(float(cum[m - 2]) - float(thr)))
    gaps.append(abs(float(cum[pick]) - float(target)))
    if pick >= 1:
        gaps.append(abs(float(cum[pick - 1]) - float(target)))
    mass_gap = min(gaps) / float(total)
    # candidates whose values nearly tie with the pick's may come in the
    # other order from logits that differ by rounding: the draw then lands on
    # the same rank but another code
    nb = [abs(float(vals[pick]) - float(vals[j])) for j in (pick - 1, pick + 1) if 0 <= j < k]
    order_gap = min(nb) if nb else np.inf
    info = {"candidates": cand, "probs": w, "cum": cum, "kept": m, "pick": pick,
            "logit_gap": logit_gap, "mass_gap": mass_gap, "order_gap": order_gap}
    return int(cand[pick]), info


def window_history(ring, pos, k, lo, window):
    """Codes of codebook k at frame positions max(lo, pos - window) .. pos - 1
    of a committed-code ring [positions][codebooks]."""
    start = max(lo, pos - window)
    return [int(ring[q][k]) for q in range(start, pos)]
