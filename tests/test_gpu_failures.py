"""Failure detection and repeatability on the GPU.

A NaN planted in one row of the fast head's weights makes that codebook
entry's logit non-finite in every fast pass: the context's non-finite counter
must see it after the frames (read by dar_nonfinite), the argmax must never
pick the entry (NaN counts as -infinity), and dar_reset must clear the
counter. Batch 1 (register kernels, one-workgroup commit) and a lockstep batch
of two (GEMM head, per-row commit).

Argmax ties: two identical rows of the fast head whose logit dominates give
bit-equal logits, and the commit picks the lower index (the oracle's np.argmax
rule), in the one-workgroup commit and in the per-row batched commit.

A paged context running the same schedule of joins and frames twice, in two
fresh contexts, returns bit-identical codes and logits (every split-K sum is
reduced in a fixed order; no float atomics).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

BF16_QNAN = 0x7FC0


@pytest.fixture(scope="module")
def tiny_host():
    d = synth.DIMS["tiny"]
    return d, synth.gen_weights(d, 0)


@pytest.mark.parametrize("batch", [1, 2])
def test_nan_weight_sets_the_nonfinite_counter(tiny_host, batch):
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    row = 17
    bad = dict(host)
    head = np.array(host["fast.head"], copy=True)
    head.view(np.uint16)[row, 0] = BF16_QNAN
    bad["fast.head"] = head
    sess = DarSession(dims, DeviceWeights(dims, bad, "bf16"), 32, batch=batch)
    prompts = [synth.gen_prompt(8 + 3 * b, dims.vocab_c0, 40 + b) for b in range(batch)]
    frames = [sess.prefill(prompts[0] if batch == 1 else prompts)]
    frames += [sess.decode_frame() for _ in range(2)]
    assert sess.nonfinite() > 0
    for codes, logits in frames:
        codes = np.asarray(codes).reshape(batch, -1)
        logits = np.asarray(logits).reshape(batch, dims.n_res + 1, -1)
        assert np.all(codes[:, 1:] != row)
        assert np.all(np.isnan(logits[:, 1:, row]))
        assert np.all(np.isfinite(logits[:, 1:, :dims.vocab_res][:, :, np.arange(dims.vocab_res) != row]))
    sess.reset()
    assert sess.nonfinite() == 0
    sess.close()


def test_paged_runs_repeat_bit_for_bit(tiny_host):
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    weights = DeviceWeights(dims, host, "bf16")
    prompts = [synth.gen_prompt(n, dims.vocab_c0, 60 + n) for n in (70, 9, 33)]

    def run():
        sess = DarSession(dims, weights, 160, batch=3, paging=(64, 8))
        out = []
        sess.seq_add(0, prompts[0])
        sess.seq_add(2, prompts[1])
        for _ in range(4):
            out.append(sess.decode_frame())
        sess.seq_add(1, prompts[2])
        for _ in range(6):
            out.append(sess.decode_frame())
        sess.seq_remove(2)
        for _ in range(3):
            out.append(sess.decode_frame())
        sess.close()
        return out

    a, b = run(), run()
    busy = [[0, 2]] * 4 + [[0, 1, 2]] * 6 + [[0, 1]] * 3  # rows of free slots are undefined
    assert len(a) == len(b) == len(busy)
    for (ca, la), (cb, lb), rows in zip(a, b, busy):
        assert np.array_equal(ca[rows], cb[rows])
        assert np.array_equal(la[rows].view(np.uint32), lb[rows].view(np.uint32))


def test_out_of_range_prompt_id_is_clamped_and_counted(tiny_host):
    """Prompt ids are not range-checked on the host: an id past the table is
    clamped to its last row (the run equals the one with that id replaced) and
    counted with the anomalies dar_nonfinite reports."""
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    weights = DeviceWeights(dims, host, "bf16")
    prompt = synth.gen_prompt(10, dims.vocab_c0, 77)
    bad, clamped = prompt.copy(), prompt.copy()
    bad[4] = dims.vocab_c0 + 5
    clamped[4] = dims.vocab_c0 - 1
    out = []
    for p in (bad, clamped):
        sess = DarSession(dims, weights, 32)
        frames = [sess.prefill(p)] + [sess.decode_frame() for _ in range(2)]
        out.append((frames, sess.nonfinite()))
        sess.close()
    (fa, na), (fb, nb) = out
    assert na == 1 and nb == 0
    for (ca, la), (cb, lb) in zip(fa, fb):
        assert np.array_equal(ca, cb)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))


@pytest.mark.parametrize("batch", [1, 3])
def test_argmax_ties_pick_the_lower_index(tiny_host, batch):
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    lo, hi, neg = 5, 9, 12
    tied = dict(host)
    head = np.array(host["fast.head"], copy=True)
    bits = head.view(np.uint16)
    bits[lo, :] = 0x3F80   # +1.0: logit = sum of the normalised input, far above the other rows
    bits[hi, :] = 0x3F80
    bits[neg, :] = 0xBF80  # -1.0: wins when that sum is negative
    tied["fast.head"] = head
    sess = DarSession(dims, DeviceWeights(dims, tied, "bf16"), 32, batch=batch)
    prompts = [synth.gen_prompt(6 + 2 * b, dims.vocab_c0, 90 + b) for b in range(batch)]
    frames = [sess.prefill(prompts[0] if batch == 1 else prompts)]
    frames += [sess.decode_frame() for _ in range(3)]
    seen = set()
    for codes, logits in frames:
        codes = np.asarray(codes).reshape(batch, -1)[:, 1:]
        logits = np.asarray(logits).reshape(batch, dims.n_res + 1, -1)[:, 1:, :]
        assert np.array_equal(logits[..., lo].view(np.uint32), logits[..., hi].view(np.uint32))
        assert np.all((codes == lo) | (codes == neg)), codes
        seen.update(np.unique(codes).tolist())
    assert lo in seen
    sess.close()


def test_ring_bounds_checked_in_64_bits_and_profile_frame_advances_position(tiny_host):
    """dar_codes rejects a range whose end overflows int32 (first near
    INT32_MAX) before any HIP call, and dar_profile_frame advances the
    position dar_position reports exactly as dar_decode_frame does."""
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights
    dims, host = tiny_host
    sess = DarSession(dims, DeviceWeights(dims, host, "bf16"), 32)
    prompt = synth.gen_prompt(8, dims.vocab_c0, 7)
    sess.prefill(prompt)
    assert sess.position() == 8
    sess.decode_frame()
    assert sess.position() == 9
    sess.profile_frame()
    assert sess.position() == 10
    sess.decode_frame()
    assert sess.position() == 11
    import torch
    dst = torch.zeros(33 * (dims.n_res + 1), dtype=torch.int32, device="cuda")
    for first, count in [(2 ** 31 - 1, 1), (2 ** 31 - 16, 32), (1, 2 ** 31 - 1), (-1, 1), (0, -1), (0, 33)]:
        with pytest.raises(N.DarError) as e:
            N.dar_codes(sess.ctx, first, count, dst.data_ptr())
        assert e.value.status == N.DAR_E_INVAL
    assert sess.ring(8, 3).shape == (3, dims.n_res + 1)
    sess.close()
