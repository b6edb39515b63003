"""Pins of the oracle's sampler (oracle/sampling.py) against hand-worked
cases, limits that reduce it to greedy argmax, the inverse-CDF property of
the draw (frequencies over an even grid of draws equal the kept
probabilities) and the decoder's use of it (window contents, greedy limit)."""
import math

import numpy as np
import pytest

import synth
from oracle import OracleDecoder, OracleModel, greedy_argmax
from oracle.sampling import SamplingParams, penalise, sample_code, window_history


def test_penalty_hand_example():
    # positive logits are divided, negative multiplied, each listed code once;
    # codes outside the vocabulary are ignored
    got = penalise([2.0, -1.0, 0.5, 3.0], [0, 1, 0, 7, -1], 2.0)
    assert got.tolist() == [1.0, -2.0, 0.5, 3.0]


def test_top_p_hand_example():
    # codes 1, 2, 0 hold 0.5, 0.3, 0.2: top-p 0.6 keeps the first two (0.5 <
    # 0.6, 0.8 >= 0.6), so draws below 0.5 / 0.8 = 0.625 give code 1, others code 2
    logits = np.log(np.array([0.2, 0.5, 0.3], dtype=np.float64)).astype(np.float32)
    p = SamplingParams(temperature=1.0, top_k=3, top_p=0.6)
    assert sample_code(logits, [], p, 0.0)[0] == 1
    assert sample_code(logits, [], p, 0.6)[0] == 1
    assert sample_code(logits, [], p, 0.65)[0] == 2
    assert sample_code(logits, [], p, 0.999)[0] == 2
    # top-p 1 keeps all three: cumulative 0.5, 0.8, 1.0
    q = SamplingParams(temperature=1.0, top_k=3, top_p=1.0)
    assert [sample_code(logits, [], q, u)[0] for u in (0.49, 0.51, 0.79, 0.81)] == [1, 2, 2, 0]


def test_top_k_hand_example():
    # top-k 2 of (1, 3, 2, 3): the two 3s (codes 1 and 3, lower code first), equal odds
    logits = np.array([1.0, 3.0, 2.0, 3.0], dtype=np.float32)
    p = SamplingParams(temperature=1.0, top_k=2, top_p=1.0)
    assert sample_code(logits, [], p, 0.25)[0] == 1
    assert sample_code(logits, [], p, 0.75)[0] == 3
    # a top-k of 3 keeps code 2 next, with weight e^-1
    q = SamplingParams(temperature=1.0, top_k=3, top_p=1.0)
    w = np.array([1.0, 1.0, math.exp(-1.0)])
    edge = (w[0] + w[1]) / w.sum()
    assert sample_code(logits, [], q, edge - 1e-4)[0] == 3
    assert sample_code(logits, [], q, edge + 1e-4)[0] == 2


@pytest.mark.parametrize("seed", range(5))
def test_greedy_limits(seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(500).astype(np.float32)
    hist = rng.integers(0, 500, 6).tolist()
    pen = penalise(logits, hist, 1.7)
    best = greedy_argmax(pen)
    for u in (0.0, 0.3, 0.999):
        # a single candidate
        assert sample_code(logits, hist, SamplingParams(0.8, 1, 1.0, 1.7, 6), u)[0] == best
        # a vanishing top-p keeps only the most probable candidate
        assert sample_code(logits, hist, SamplingParams(0.8, 64, 1e-7, 1.7, 6), u)[0] == best


def test_draw_direction_and_flat_limit():
    # equal logits: the candidates are codes 0..k-1 in order and each holds
    # 1/k of the mass, so draw u falls on candidate floor(u k)
    logits = np.zeros(300, dtype=np.float32)
    p = SamplingParams(temperature=1.0, top_k=40, top_p=1.0)
    for u in np.linspace(0.0, 0.999, 37):
        assert sample_code(logits, [], p, float(u))[0] == int(np.floor(u * 40 + 1e-9))


@pytest.mark.parametrize("seed", range(4))
def test_frequencies_match_kept_probabilities(seed):
    """Over an even grid of N draws the code frequencies are the truncated,
    renormalised softmax (computed here in fp64 by enumerating the kept set)."""
    rng = np.random.default_rng(100 + seed)
    V = 257
    logits = (rng.standard_normal(V) * 2.0).astype(np.float32)
    hist = rng.integers(0, V, 10).tolist()
    p = SamplingParams(temperature=0.7, top_k=37, top_p=0.85, penalty=1.3, window=10)
    # fp64 enumeration of the kept set
    v = logits.astype(np.float64).copy()
    for c in set(hist):
        v[c] = v[c] / 1.3 if v[c] > 0 else v[c] * 1.3
    v = v / 0.7
    ranked = sorted(range(V), key=lambda j: (-v[j], j))[:37]
    e = np.array([math.exp(v[j] - v[ranked[0]]) for j in ranked])
    prob = e / e.sum()
    n_keep = int(np.searchsorted(np.cumsum(prob), 0.85)) + 1
    kept = ranked[:n_keep]
    q = prob[:n_keep] / prob[:n_keep].sum()
    N = 20000
    counts = {}
    for i in range(N):
        c = sample_code(logits, hist, p, (i + 0.5) / N)[0]
        counts[c] = counts.get(c, 0) + 1
    assert set(counts) <= set(kept)
    for j, qj in zip(kept, q):
        assert abs(counts.get(j, 0) / N - qj) <= 1.0 / N + 1e-5, (j, counts.get(j, 0) / N, qj)


def test_window_history():
    ring = np.array([[9, 9], [1, 5], [2, 6], [3, 7], [4, 8]])
    # frames start at position 1; window 2 at position 4 reads positions 2, 3
    assert window_history(ring, 4, 1, 1, 2) == [6, 7]
    # a window longer than the generated frames stops at the first frame
    assert window_history(ring, 3, 0, 1, 10) == [1, 2]
    assert window_history(ring, 1, 0, 1, 4) == []


@pytest.fixture(scope="module")
def tiny():
    d = synth.DIMS["tiny"]
    return d, OracleModel(d, synth.gen_weights(d, 0))


def test_decoder_top1_sampling_is_greedy(tiny):
    d, m = tiny
    prompt = synth.gen_prompt(8, d.vocab_c0, 3)
    u = np.random.default_rng(5).random((40, d.n_res + 1))
    g = OracleDecoder(m, 40)
    s = OracleDecoder(m, 40, SamplingParams(temperature=0.5, top_k=1, top_p=1.0), u)
    a = [g.prefill(prompt)] + [g.decode_frame() for _ in range(4)]
    b = [s.prefill(prompt)] + [s.decode_frame() for _ in range(4)]
    for (ca, la), (cb, lb) in zip(a, b):
        assert np.array_equal(ca, cb)
        for x, y in zip(la, lb):
            assert np.array_equal(x, y)


def test_decoder_ring_and_window(tiny):
    """The ring holds the committed codes (forced ones when forced) at each
    frame's slow position, and each draw's window reads exactly them."""
    d, m = tiny
    prompt = synth.gen_prompt(6, d.vocab_c0, 4)
    rng = np.random.default_rng(6)
    u = rng.random((30, d.n_res + 1))
    params = SamplingParams(temperature=0.9, top_k=20, top_p=0.9, penalty=1.5, window=3)
    forced = [np.concatenate([[rng.integers(d.vocab_c0)], rng.integers(0, d.vocab_res, d.n_res)]) for _ in range(6)]
    dec = OracleDecoder(m, 30, params, u)
    frames = [dec.prefill(prompt, forced=forced[0])] + [dec.decode_frame(forced=forced[i]) for i in range(1, 6)]
    for i in range(6):
        assert np.array_equal(dec.ring[5 + i], forced[i])
    # replay frame 4 (position 9) codebook 2 by hand: window positions 6..8
    codes, logits = frames[4]
    hist = [int(forced[j][2]) for j in (1, 2, 3)]
    want, _ = sample_code(logits[2], hist, params, float(u[9][2]))
    assert codes[2] == want
