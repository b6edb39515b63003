"""Batched decode (several sequences in lockstep, ragged prompt lengths).

Tiny Dual-AR (2 slow layers, 1 fast layer, d 256): each sequence of the batch
is teacher-forced with its own oracle greedy frames and compared with its own
oracle run (logits rel-L2, argmax agreement, exact codes above the margin),
bf16, fp8, int8 and int4 at B = 4, at the largest batch (64, whose first fast
pass is a 128-row GEMM; bf16 and int4) and with prompts long enough for several
attention splits. At full shape (36 + 4 layers, d 2560): a batch of two equals
two batch-1 contexts decoding the same prompts (same codes where the margin
exceeds 1e-2, logits within the bf16 tolerance).
"""
import numpy as np
import pytest

import synth
from oracle import OracleDecoder, OracleModel
from parity import TOL, assert_parity, compare_frames

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_host():
    d = synth.DIMS["tiny"]
    return d, synth.gen_weights(d, 0)


def _oracle_frames(model, prompt, frames, max_len):
    dec = OracleDecoder(model, max_len)
    out = [dec.prefill(prompt)]
    for _ in range(frames):
        out.append(dec.decode_frame())
    return out


# the last case spans several 64-position attention splits, with the longest
# sequence crossing a split boundary while the frames are decoded
@pytest.mark.parametrize("wtype,B,frames,max_len,lmax",
                         [("bf16", 4, 20, 48, 24), ("fp8", 4, 20, 48, 24), ("int8", 4, 20, 48, 24),
                          ("int4", 4, 20, 48, 24), ("bf16", 64, 2, 48, 24), ("int4", 64, 2, 48, 24),
                          ("bf16", 3, 24, 200, 130)])
def test_tiny_batched_parity(tiny_host, wtype, B, frames, max_len, lmax):
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(4, lmax, B)]
    if lmax > 64:
        lens[0] = lmax - 10  # frames take it across position 128
    prompts = [synth.gen_prompt(n, dims.vocab_c0, 100 + b) for b, n in enumerate(lens)]
    model = OracleModel(dims, host, wtype=wtype)
    refs = [_oracle_frames(model, p, frames, max_len) for p in prompts]
    sess = DarSession(dims, DeviceWeights(dims, host, wtype), max_len, batch=B)
    forced = [np.stack([refs[b][i][0] for b in range(B)]) for i in range(frames + 1)]
    got = [sess.prefill(prompts, forced=forced[0])]
    for i in range(1, frames + 1):
        got.append(sess.decode_frame(forced=forced[i]))
    stats_all = {"max_rel": 0.0, "agree": 0.0, "n": 0, "exact_fail": [], "tol": TOL[wtype]}
    for b in range(B):
        gb = [(codes[b], logits[b]) for codes, logits in got]
        st = compare_frames(gb, refs[b], dims, wtype)
        stats_all["max_rel"] = max(stats_all["max_rel"], st["max_rel"])
        stats_all["agree"] += st["agree"] * st["n"]
        stats_all["n"] += st["n"]
        stats_all["exact_fail"] += [(b,) + e for e in st["exact_fail"]]
    stats_all["agree"] /= stats_all["n"]
    print(f"\n{wtype} B={B}: {stats_all}")
    assert_parity(stats_all)
    assert sess.position() == [n + frames for n in lens]
    ring = sess.ring(0, max_len)
    for b in range(B):
        for i in range(frames + 1):
            assert np.array_equal(ring[lens[b] - 1 + i, b], forced[i][b])
    assert sess.nonfinite() == 0
    sess.close()


def test_batched_capacity_and_errors(tiny_host):
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    sess = DarSession(dims, DeviceWeights(dims, host, "bf16"), 16, batch=3)
    # the batch decodes in lockstep: a prefill must bring one prompt per sequence
    with pytest.raises(N.DarError) as e:
        N.dar_prefill(sess.ctx, 2, 0, [4, 5], None, None, None)
    assert e.value.status == N.DAR_E_INVAL
    prompts = [synth.gen_prompt(n, dims.vocab_c0, n) for n in (3, 9, 14)]
    sess.prefill(prompts, want=False)   # frame 0 at positions 2, 8, 13
    sess.decode_frame(want=False)       # 3, 9, 14
    sess.decode_frame(want=False)       # 4, 10, 15: the longest sequence reaches max_len - 1
    assert sess.position() == [5, 11, 16]
    with pytest.raises(N.DarError) as e:
        sess.decode_frame(want=False)
    assert e.value.status == N.DAR_E_CAPACITY
    sess.close()


def test_fullshape_batch_equals_single():
    import torch

    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    wl = synth.WORKLOADS["s2pro_dual_bf16"]
    dims = wl.dims
    host = synth.gen_weights(dims, wl.weight_seed)
    dw = DeviceWeights(dims, host, "bf16")
    del host
    prompts = [synth.gen_prompt(n, dims.vocab_c0, 50 + n) for n in (128, 160)]
    frames, max_len = 4, 256
    single = []
    for p in prompts:
        s1 = DarSession(dims, dw, max_len)
        out = [s1.prefill(p)]
        for _ in range(frames):
            out.append(s1.decode_frame())
        single.append(out)
        s1.close()
    # the batch is forced with the single runs' own codes, so that a near-tie
    # resolved differently cannot change the later inputs
    forced = [np.stack([single[b][i][0] for b in range(2)]) for i in range(frames + 1)]
    sb = DarSession(dims, dw, max_len, batch=2)
    got = [sb.prefill(prompts, forced=forced[0])]
    for i in range(1, frames + 1):
        got.append(sb.decode_frame(forced=forced[i]))
    sb.close()
    for b in range(2):
        gb = [(codes[b], logits[b]) for codes, logits in got]
        st = compare_frames(gb, single[b], dims, "bf16")
        print(f"\nsequence {b}: {st}")
        assert st["max_rel"] <= TOL["bf16"], st
        assert not st["exact_fail"], st
    del dw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["s2pro_dual_b16", "s2pro_dual_b64"])
def test_fullshape_lockstep_batch_matches_oracle(name):
    """Full shape in the batched benchmark's configuration (16 or 64 sequences
    decoded in lockstep, max length 4096, ragged prompts of 128..512 ids): row
    0 holds the stored oracle reference runs (prefill 128 + 9 greedy-forced
    frames, and the frame at position 1007 after 880 randomly forced frames)
    beside the workload's own prompts in the other rows; row 0's frames must
    meet the full-shape bar (whole logit vectors within the bf16 relative-L2
    tolerance, codes exact above the 1e-2 margin, >= 99% agreement)."""
    import torch

    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    from test_gpu_fullshape import _compare, _golden, _random_frames
    wl = synth.WORKLOADS[name]
    ref_wl = synth.WORKLOADS["s2pro_dual_bf16"]
    dims = wl.dims
    B = wl.batch
    ref = _golden(ref_wl.name)
    host = synth.gen_weights(dims, wl.weight_seed)
    dw = DeviceWeights(dims, host, "bf16")
    del host
    lens, prompts = synth.gen_ragged_prompts(B, wl.prefill_len, wl.prefill_len_max, dims.vocab_c0,
                                             wl.prompt_seed, wl.length_seed)
    prompts = [synth.gen_prompt(ref_wl.prefill_len, dims.vocab_c0, ref_wl.prompt_seed)] + list(prompts[1:])
    sess = DarSession(dims, dw, wl.max_len, batch=B)
    fc = dims.n_res + 1
    rng = np.random.default_rng(31)
    stats = {"rel": [], "n": 0, "agree": 0, "exact_fail": []}

    def run(row0_frames, keep):
        outs = []
        for i, f in enumerate(row0_frames):
            forced = rng.integers(0, min(dims.vocab_c0, dims.vocab_res), (B, fc)).astype(np.int32)
            forced[0] = f
            if i == 0:
                out = sess.prefill(prompts, forced=forced, want=keep(i))
            else:
                out = sess.decode_frame(forced=forced, want=keep(i))
            if keep(i):
                outs.append((out[0][0].copy(), out[1][0].copy()))
        return outs

    early = [np.asarray(f, dtype=np.int32) for f in ref["early"]["forced"]]
    got = run(early, lambda i: True)
    for (codes, logits), rv, rf in zip(got, ref["early"]["frames"], ref["early"]["full"]):
        _compare(rv, rf, codes, logits, dims, stats)
    late = ref["late"]
    forced = [np.asarray(f, dtype=np.int32) for f in _random_frames()(dims, late["frames_forced"], late["force_seed"])]
    got = run(forced, lambda i: i == len(forced) - 1)
    assert sess.position()[0] == late["position"] + 1
    codes, logits = got[-1]
    _compare(late["frame"], late["full"], codes, logits, dims, stats)
    agree = stats["agree"] / stats["n"]
    print(f"\nlockstep full shape B={B}: max rel {max(stats['rel']):.3e}, median rel {np.median(stats['rel']):.3e}, "
          f"agreement {agree:.4f} over {stats['n']} vectors, exact failures {stats['exact_fail']}")
    assert max(stats["rel"]) <= TOL["bf16"], stats
    assert not stats["exact_fail"], stats
    assert agree >= 0.99, stats
    assert sess.nonfinite() == 0
    sess.close()
    del dw
    torch.cuda.empty_cache()
