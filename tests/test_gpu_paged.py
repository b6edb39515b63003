"""Continuous batching over a paged slow KV cache (dar_create_paged).

Tiny Dual-AR (2 slow layers, 1 fast layer, d 256), four slots, pages of 64
positions. Sequences join and leave while the others keep decoding. A
sequence that joins takes pages another one just returned (stale KV in them).
One slot stays free throughout (its parked rows run every frame). Prompts
span several pages, and sequences cross page boundaries while decoding.
Every sequence is teacher-forced with its own oracle greedy frames and held to
the bar of a single sequence: logits rel-L2, argmax agreement, exact codes
above the margin (bf16, fp8, int8, int4, and bf16 with graph replay). Sampling
draws from each slot's uniforms with its own repetition window. Pool
exhaustion and the position limit return DAR_E_CAPACITY and change nothing:
the run continues after a removal and still matches the oracle. At full shape,
in the continuous-batching bench's configuration, one slot beside three other
sequences meets the full-shape bar against the stored oracle references for
every weight type.
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


class Driver:
    """Runs a schedule of adds, removes and frames on a paged session, forcing
    each slot's sequence with its oracle frames and collecting its outputs."""

    def __init__(self, sess, dims, refs):
        self.sess, self.dims, self.refs = sess, dims, refs
        self.fc = dims.n_res + 1
        self.slot_seq = {}                     # slot -> sequence id
        self.done = {k: 0 for k in refs}       # frames returned per sequence
        self.got = {k: [] for k in refs}

    def add(self, slot, seq, prompt):
        self.sess.seq_add(slot, prompt)
        self.slot_seq[slot] = seq

    def remove(self, slot):
        self.sess.seq_remove(slot)
        del self.slot_seq[slot]

    def frame(self):
        forced = np.zeros((self.sess.batch, self.fc), dtype=np.int32)
        for slot, seq in self.slot_seq.items():
            forced[slot] = self.refs[seq][self.done[seq]][0]
        codes, logits = self.sess.decode_frame(forced=forced)
        for slot, seq in self.slot_seq.items():
            self.got[seq].append((codes[slot].copy(), logits[slot].copy()))
            self.done[seq] += 1

    def check(self, wtype):
        allst = {"max_rel": 0.0, "agree": 0.0, "n": 0, "exact_fail": [], "tol": TOL[wtype]}
        for seq, frames in self.got.items():
            st = compare_frames(frames, self.refs[seq][:len(frames)], self.dims, wtype)
            allst["max_rel"] = max(allst["max_rel"], st["max_rel"])
            allst["agree"] += st["agree"] * st["n"]
            allst["n"] += st["n"]
            allst["exact_fail"] += [(seq,) + e for e in st["exact_fail"]]
        allst["agree"] /= allst["n"]
        return allst


@pytest.mark.parametrize("wtype,graph", [("bf16", False), ("fp8", False), ("int8", False), ("int4", False),
                                         ("bf16", True)])
def test_paged_continuous_parity(tiny_host, wtype, graph):
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    max_len, page, n_pages = 200, 64, 12
    lens = {"A": 60, "B": 20, "C": 130, "D": 5, "E": 100}
    frames = {"A": 16, "B": 6, "C": 20, "D": 14, "E": 8}
    prompts = {k: synth.gen_prompt(n, dims.vocab_c0, 300 + i) for i, (k, n) in enumerate(lens.items())}
    model = OracleModel(dims, host, wtype=wtype)
    refs = {k: _oracle_frames(model, prompts[k], frames[k], max_len) for k in lens}
    sess = DarSession(dims, DeviceWeights(dims, host, wtype), max_len, batch=4, paging=(page, n_pages), graph=graph)
    assert sess.pages_free() == n_pages - 1
    drv = Driver(sess, dims, refs)
    drv.add(0, "A", prompts["A"])      # 1 page; crosses into its second page at its 5th frame
    drv.add(2, "B", prompts["B"])      # 1 page
    assert sess.pages_free() == n_pages - 3
    for _ in range(3):
        drv.frame()
    drv.add(1, "C", prompts["C"])      # 3 pages, attention over three splits
    for _ in range(4):
        drv.frame()
    assert sess.position() == [lens["A"] - 1 + 7, lens["C"] - 1 + 4, lens["B"] - 1 + 7, -1]
    drv.remove(2)                      # B leaves after 7 frames; D reuses its page (stale KV)
    drv.add(2, "D", prompts["D"])
    for _ in range(6):
        drv.frame()
    drv.remove(0)                      # A leaves after 13 frames
    drv.add(0, "E", prompts["E"])
    for _ in range(9):
        drv.frame()                    # E: frames 0..8
    st = drv.check(wtype)
    print(f"\n{wtype} paged: {st}")
    assert_parity(st)
    assert {k: len(v) for k, v in drv.got.items()} == {"A": 13, "B": 7, "C": 19, "D": 15, "E": 9}
    for slot in list(drv.slot_seq):
        drv.remove(slot)
    assert sess.pages_free() == n_pages - 1
    assert sess.position() == [-1, -1, -1, -1]
    assert sess.nonfinite() == 0
    sess.close()


def test_paged_sampling_matches_oracle(tiny_host):
    """Sampling in a paged context: each sequence draws from the uniforms of
    its slot at its own frame positions and its repetition window starts at
    its own first frame, also in a slot whose previous sequence left codes in
    the committed-code ring at the positions it reaches."""
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    from test_gpu_sampling import PARAMS, _check_codes
    dims, host = tiny_host
    fc = dims.n_res + 1
    max_len, S = 64, 4
    u = synth.gen_uniforms(max_len, S, fc, 13)
    spec = {"P": (0, 12, 18), "X": (1, 30, 6), "Q": (2, 5, 15), "Y": (1, 10, 12)}  # slot, prompt, frames
    prompts = {k: synth.gen_prompt(n, dims.vocab_c0, 500 + i) for i, (k, (_, n, _)) in enumerate(spec.items())}
    model = OracleModel(dims, host, "bf16")
    refs, margins = {}, {}
    for k, (slot, n, f) in spec.items():
        dec = OracleDecoder(model, max_len, PARAMS, u[:, slot, :])
        refs[k] = [dec.prefill(prompts[k])] + [dec.decode_frame() for _ in range(f - 1)]
        margins[k] = dec.margins
    sess = DarSession(dims, DeviceWeights(dims, host, "bf16"), max_len, batch=S, paging=(64, 8))
    sess.set_sampling(PARAMS.temperature, PARAMS.top_k, PARAMS.top_p, PARAMS.penalty, PARAMS.window, u)
    drv = Driver(sess, dims, refs)
    drv.add(0, "P", prompts["P"])
    drv.add(1, "X", prompts["X"])
    for _ in range(3):
        drv.frame()
    drv.add(2, "Q", prompts["Q"])
    for _ in range(3):
        drv.frame()
    drv.remove(1)                      # X leaves after 6 frames; Y reuses its slot and ring column
    drv.add(1, "Y", prompts["Y"])
    for _ in range(12):
        drv.frame()
    assert {k: len(v) for k, v in drv.got.items()} == {k: f for k, (_, _, f) in spec.items()}
    for k in spec:
        agree, total, unsafe = _check_codes(drv.got[k], refs[k], margins[k], dims)
        print(f"\n{k}: sampled codes agree {agree}/{total} ({unsafe} within rounding of a boundary)")
    sess.close()


def test_paged_capacity_changes_nothing(tiny_host):
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    max_len, page, n_pages = 256, 64, 4        # 3 usable pages
    lens = {"A": 62, "B": 64, "C": 10}
    frames = {"A": 8, "B": 4, "C": 4}
    prompts = {k: synth.gen_prompt(n, dims.vocab_c0, 400 + i) for i, (k, n) in enumerate(lens.items())}
    model = OracleModel(dims, host, wtype="bf16")
    refs = {k: _oracle_frames(model, prompts[k], frames[k], max_len) for k in lens}
    sess = DarSession(dims, DeviceWeights(dims, host, "bf16"), max_len, batch=2, paging=(page, n_pages))
    drv = Driver(sess, dims, refs)
    # a prompt longer than the pool, and an occupied slot, are refused
    long_prompt = synth.gen_prompt(200, dims.vocab_c0, 9)
    with pytest.raises(N.DarError) as e:
        sess.seq_add(0, long_prompt)
    assert e.value.status == N.DAR_E_CAPACITY
    assert sess.pages_free() == 3
    drv.add(0, "A", prompts["A"])      # positions 0..61: page 1
    drv.add(1, "B", prompts["B"])      # positions 0..63: one page; its first slow step needs a second
    with pytest.raises(N.DarError) as e:
        sess.seq_add(1, prompts["C"])
    assert e.value.status == N.DAR_E_STATE
    assert sess.pages_free() == 1
    drv.frame()                        # B's slow step at 64 takes the last page
    assert sess.pages_free() == 0
    drv.frame()                        # A's slow step at 62..63: still its first page
    with pytest.raises(N.DarError) as e:
        drv.frame()                    # A's slow step at 64 needs a page: refused, nothing changes
    assert e.value.status == N.DAR_E_CAPACITY
    assert sess.position() == [lens["A"] - 1 + 2, lens["B"] - 1 + 2]
    drv.remove(1)                      # B leaves: two pages back
    drv.add(1, "C", prompts["C"])
    for _ in range(4):
        drv.frame()
    st = drv.check("bf16")
    print(f"\npaged capacity run: {st}")
    assert_parity(st)
    assert {k: len(v) for k, v in drv.got.items()} == {"A": 6, "B": 2, "C": 4}
    sess.close()


def test_paged_position_limit(tiny_host):
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    sess = DarSession(dims, DeviceWeights(dims, host, "bf16"), 64, batch=2, paging=(64, 3))
    sess.seq_add(1, synth.gen_prompt(60, dims.vocab_c0, 5))   # frame 0 at 59
    for _ in range(3):
        sess.decode_frame(want=False)                        # frames at 59, 60, 61; next at 62 = max_len - 2
    sess.decode_frame(want=False)
    assert sess.position() == [-1, 63]
    with pytest.raises(N.DarError) as e:
        sess.decode_frame(want=False)                        # its slow step would be at 64 = max_len
    assert e.value.status == N.DAR_E_CAPACITY
    sess.seq_remove(1)
    with pytest.raises(N.DarError) as e:
        sess.decode_frame(want=False)                        # no sequence left
    assert e.value.status == N.DAR_E_STATE
    with pytest.raises(N.DarError) as e:
        sess.seq_remove(1)                                   # already free
    assert e.value.status == N.DAR_E_STATE
    for slot in (-1, 2):
        with pytest.raises(N.DarError) as e:
            sess.seq_add(slot, synth.gen_prompt(4, dims.vocab_c0, 6))
        assert e.value.status == N.DAR_E_INVAL
        with pytest.raises(N.DarError) as e:
            sess.seq_remove(slot)
        assert e.value.status == N.DAR_E_INVAL
    with pytest.raises(N.DarError) as e:
        sess.seq_add(0, synth.gen_prompt(64, dims.vocab_c0, 7))   # len == max_len
    assert e.value.status == N.DAR_E_CAPACITY
    assert sess.pages_free() == 2
    # a paged context takes no lockstep prefill
    with pytest.raises(N.DarError) as e:
        sess.prefill([synth.gen_prompt(4, dims.vocab_c0, 8)] * 2, want=False)
    assert e.value.status == N.DAR_E_STATE
    sess.close()


@pytest.mark.parametrize("name", ["s2pro_dual_bf16", "s2pro_dual_fp8", "s2pro_dual_int8", "s2pro_dual_int4"])
def test_fullshape_paged_matches_oracle(name):
    """Full shape (36 + 4 layers, d 2560; bf16, fp8, int8, int4) in the continuous-batching
    bench's configuration (16 slots, 256-position pages, 97 pages, max length
    4096): one slot decodes the oracle reference runs while three other slots
    hold other sequences; its frames must meet the full-shape bar against the
    stored oracle references (prefill 128 + 9 greedy-forced frames, and the
    frame at position 1007 after 880 randomly forced frames)."""
    import torch

    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    from test_gpu_fullshape import _compare, _golden, _random_frames
    wl = synth.WORKLOADS[name]
    cb = synth.WORKLOADS["s2pro_dual_cb16"]
    dims = wl.dims
    ref = _golden(name)
    host = synth.gen_weights(dims, wl.weight_seed)
    dw = DeviceWeights(dims, host, wl.wtype)
    del host
    sess = DarSession(dims, dw, cb.max_len, batch=cb.batch, paging=(cb.page_len, cb.n_pages))
    prompt = synth.gen_prompt(wl.prefill_len, dims.vocab_c0, wl.prompt_seed)
    others = {b: synth.gen_prompt(300, dims.vocab_c0, 600 + b) for b in (0, 1, 2)}
    slot = 5
    fc = dims.n_res + 1
    stats = {"rel": [], "n": 0, "agree": 0, "exact_fail": []}

    def run(forced_frames, keep):
        for b, p in others.items():
            sess.seq_add(b, p)
        sess.seq_add(slot, prompt)
        outs = []
        for i, f in enumerate(forced_frames):
            forced = np.zeros((cb.batch, fc), dtype=np.int32)
            forced[slot] = f
            out = sess.decode_frame(forced=forced, want=keep(i))
            if keep(i):
                outs.append((out[0][slot].copy(), out[1][slot].copy()))
        return outs

    early = [np.asarray(f, dtype=np.int32) for f in ref["early"]["forced"]]
    got = run(early, lambda i: True)
    for (codes, logits), rv, rf in zip(got, ref["early"]["frames"], ref["early"]["full"]):
        _compare(rv, rf, codes, logits, dims, stats)
    sess.reset()
    assert sess.pages_free() == cb.n_pages - 1
    late = ref["late"]
    forced = [np.asarray(f, dtype=np.int32) for f in _random_frames()(dims, late["frames_forced"], late["force_seed"])]
    got = run(forced, lambda i: i == len(forced) - 1)
    assert sess.position()[slot] == late["position"] + 1
    codes, logits = got[-1]
    _compare(late["frame"], late["full"], codes, logits, dims, stats)
    agree = stats["agree"] / stats["n"]
    print(f"\npaged full shape {name}: max rel {max(stats['rel']):.3e}, agreement {agree:.4f} over {stats['n']} "
          f"vectors, exact failures {stats['exact_fail']}")
    assert max(stats["rel"]) <= TOL[wl.wtype], stats
    assert not stats["exact_fail"], stats
    assert agree >= 0.99, stats
    assert sess.nonfinite() == 0
    sess.close()
    del dw
    torch.cuda.empty_cache()
