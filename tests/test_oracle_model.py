"""Pins for the oracle's whole-model paths.

* KV-cached decode equals a cache-free causal recompute, for the slow AR over a
  whole prompt+decode sequence and for the fast AR inside each frame (this ties
  cache writes, positions, causality and the fast sequence layout together).
* Prefill as one causal block equals prefill one token at a time.
* Reduced models with a closed-form answer: with every Wo and W2 zero, the
  layers are the identity on the residual and the logits are W0 . norm(W0[tok]);
  with Wq zero as well as W2, attention is a plain running mean of the values.
* fp32 and fp64 runs of the same oracle agree far inside the GPU tolerances.
* Greedy determinism, and teacher forcing with the model's own codes
  reproducing the free run.
"""
import numpy as np
import pytest

import synth
from oracle import OracleDecoder, OracleModel, bf16_to_f32, full_recompute_fast, full_recompute_slow, rmsnorm
from synth import DarDims

MICRO = DarDims(name="micro", n_layers_slow=2, n_layers_fast=2, d_model=32, n_heads_q=4, n_heads_kv=2,
                head_dim=8, ffn_dim=48, vocab_c0=50, vocab_res=20, n_res=3)


def _model(dims=MICRO, dt=np.float64, wtype="bf16", edit=None, seed=0, kv="bf16"):
    w = synth.gen_weights(dims, seed)
    if edit:
        edit(w)
    return OracleModel(dims, w, wtype=wtype, dt=dt, kv=kv), w


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b))


def _run(dec, prompt, frames, forced=None):
    out_codes, out_logits = [], []
    c, lg = dec.prefill(prompt, forced=None if forced is None else forced[0])
    out_codes.append(c)
    out_logits.append(lg)
    for i in range(1, frames + 1):
        c, lg = dec.decode_frame(forced=None if forced is None else forced[i])
        out_codes.append(c)
        out_logits.append(lg)
    return np.array(out_codes), out_logits


@pytest.mark.parametrize("dims", [MICRO, synth.DIMS["tiny"]], ids=["micro", "tiny"])
def test_cached_decode_equals_full_recompute(dims):
    m, _ = _model(dims)
    prompt = synth.gen_prompt(7, dims.vocab_c0, 3)
    dec = OracleDecoder(m, 20)
    codes, logits = _run(dec, prompt, 6)
    slow_in = np.concatenate([prompt, codes[:-1, 0]])
    l0_full, h_full = full_recompute_slow(m, slow_in)
    for f in range(7):
        p = len(prompt) - 1 + f
        assert _rel(logits[f][0], l0_full[p]) < 1e-12
        fast_full = full_recompute_fast(m, h_full[p], codes[f])
        for k in range(1, dims.n_res + 1):
            assert _rel(logits[f][k], fast_full[k - 1]) < 1e-12


def test_prefill_block_equals_token_by_token():
    m, _ = _model()
    prompt = synth.gen_prompt(9, MICRO.vocab_c0, 4)
    a = OracleDecoder(m, 16)
    b = OracleDecoder(m, 16)
    ca, la = a.prefill(prompt, block=True)
    cb, lb = b.prefill(prompt, block=False)
    assert np.array_equal(ca, cb)
    for x, y in zip(la, lb):
        assert _rel(x, y) < 1e-12
    assert np.allclose(a.k, b.k, rtol=1e-12, atol=1e-14) and np.allclose(a.v, b.v, rtol=1e-12, atol=1e-14)


def _zero(names):
    def edit(w):
        for n in names:
            w[n] = np.zeros_like(w[n])
    return edit


def test_identity_layers_reduce_to_tied_table_closed_form():
    d = MICRO
    names = [f"slow.{i}.{m}" for i in range(d.n_layers_slow) for m in ("wo", "w2")]
    m, w = _model(edit=_zero(names))
    prompt = synth.gen_prompt(5, d.vocab_c0, 5)
    dec = OracleDecoder(m, 8)
    _, logits = dec.prefill(prompt)
    w0 = bf16_to_f32(w["w0"]).astype(np.float64)
    g = bf16_to_f32(w["slow.final_norm"]).astype(np.float64)
    x = w0[prompt[-1]]
    h = g * x / np.sqrt(np.mean(x * x) + d.rms_eps)
    assert _rel(logits[0], w0 @ h) < 1e-13


def test_uniform_attention_closed_form():
    d = DarDims(name="one", n_layers_slow=1, n_layers_fast=0, d_model=32, n_heads_q=4, n_heads_kv=2,
                head_dim=8, ffn_dim=48, vocab_c0=50, vocab_res=0, n_res=0)
    qw = d.q_width

    def edit(w):
        qkv = w["slow.0.wqkv"].copy()
        qkv[:qw] = 0                        # Wq = 0: every score is 0, weights uniform
        w["slow.0.wqkv"] = qkv
        w["slow.0.w2"] = np.zeros_like(w["slow.0.w2"])
    m, w = _model(dims=d, edit=edit, kv="fp32")     # exact-math check: no storage rounding
    prompt = synth.gen_prompt(6, d.vocab_c0, 6)
    dec = OracleDecoder(m, 10)
    _, logits = dec.prefill(prompt)
    f = {k: bf16_to_f32(v).astype(np.float64) for k, v in w.items()}
    xs = f["w0"][prompt]                                            # [6, d]
    ga = f["slow.0.attn_norm"]
    wv = f["slow.0.wqkv"][qw + d.kv_width:]                         # V rows
    vs = np.array([wv @ (ga * x / np.sqrt(np.mean(x * x) + d.rms_eps)) for x in xs])  # [6, kv_width]
    mean_v = vs.mean(axis=0).reshape(d.n_heads_kv, d.head_dim)
    o = np.concatenate([mean_v[h // d.group] for h in range(d.n_heads_q)])
    x_out = xs[-1] + f["slow.0.wo"] @ o
    gf = f["slow.final_norm"]
    want = f["w0"] @ (gf * x_out / np.sqrt(np.mean(x_out * x_out) + d.rms_eps))
    assert _rel(logits[0], want) < 1e-13


def test_fp32_oracle_close_to_fp64():
    d = synth.DIMS["tiny"]
    # arithmetic precision only (with bf16 storage a rounding tie can land
    # differently in fp32 and fp64, which the next test bounds separately)
    m64, w = _model(d, np.float64, kv="fp32")
    m32 = OracleModel(d, w, dt=np.float32, kv="fp32")
    prompt = synth.gen_prompt(16, d.vocab_c0, 1)
    rng = np.random.default_rng(9)
    forced = [np.concatenate([[rng.integers(d.vocab_c0)], rng.integers(0, d.vocab_res, d.n_res)]) for _ in range(6)]
    _, l64 = _run(OracleDecoder(m64, 32), prompt, 5, forced)
    _, l32 = _run(OracleDecoder(m32, 32), prompt, 5, forced)
    worst = max(_rel(a, b) for fa, fb in zip(l32, l64) for a, b in zip(fa, fb))
    assert worst < 1e-5


def test_greedy_is_deterministic_and_self_forcing_reproduces_it():
    d = synth.DIMS["tiny"]
    m, _ = _model(d, np.float32)
    prompt = synth.gen_prompt(16, d.vocab_c0, 1)
    c1, l1 = _run(OracleDecoder(m, 32), prompt, 4)
    c2, l2 = _run(OracleDecoder(m, 32), prompt, 4)
    c3, l3 = _run(OracleDecoder(m, 32), prompt, 4, forced=c1)
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    for fa, fb, fc in zip(l1, l2, l3):
        for a, b, c in zip(fa, fb, fc):
            assert np.array_equal(a, b) and np.array_equal(a, c)


def test_forcing_changes_inputs_not_outputs_contract():
    # forced codes drive the next inputs; the returned codes are still the argmax
    d = MICRO
    m, _ = _model(d)
    prompt = synth.gen_prompt(4, d.vocab_c0, 7)
    forced = np.array([3, 1, 2, 3])
    dec = OracleDecoder(m, 8)
    codes, logits = dec.prefill(prompt, forced=forced)
    assert codes[0] == int(np.argmax(logits[0]))
    assert all(codes[k] == int(np.argmax(logits[k])) for k in range(4))
    assert dec.last_c0 == 3


def test_fp8_model_uses_dequantised_linears():
    d = MICRO
    w = synth.gen_weights(d, 0)
    m8 = OracleModel(d, w, wtype="fp8", dt=np.float64)
    codes, scale = m8.quant["slow.1.w3"]
    from oracle import e4m3_decode
    x = np.random.default_rng(1).standard_normal(d.d_model)
    want = (e4m3_decode(codes).astype(np.float64) * scale[:, None].astype(np.float64)) @ x
    assert _rel(m8.slow[1].w3(x), want) < 1e-13
    assert len(m8.quant) == len(synth.linear_names(d))
    # tables and norms are untouched by quantisation
    assert np.array_equal(m8.w0, bf16_to_f32(w["w0"]).astype(np.float64))


def test_decode_state_errors():
    m, _ = _model()
    dec = OracleDecoder(m, 5)
    with pytest.raises(RuntimeError):
        dec.decode_frame()
    dec.prefill(synth.gen_prompt(4, MICRO.vocab_c0, 1))
    dec.decode_frame()
    with pytest.raises(RuntimeError):
        dec.decode_frame()


def test_rmsnorm_used_for_fast_input_is_slow_final_norm():
    # h_t handed to the fast AR is the final-normed slow output (the head's input)
    d = MICRO
    m, _ = _model(d)
    x = np.random.default_rng(2).standard_normal(d.d_model)
    logits, h = m.head0(x)
    assert np.allclose(h, rmsnorm(x, m.slow_final_norm, d.rms_eps))
    assert np.allclose(logits, m.w0 @ h)


def test_kv_storage_precision_effect_is_bounded():
    # bf16 KV storage (the pages' activation dtype) vs fp32 storage: the logits
    # move by far less than the 2e-2 relative tolerance used for GPU parity
    d = synth.DIMS["tiny"]
    w = synth.gen_weights(d, 0)
    prompt = synth.gen_prompt(16, d.vocab_c0, 1)
    rng = np.random.default_rng(4)
    forced = [np.concatenate([[rng.integers(d.vocab_c0)], rng.integers(0, d.vocab_res, d.n_res)]) for _ in range(6)]
    _, lb = _run(OracleDecoder(OracleModel(d, w, kv="bf16"), 32), prompt, 5, forced)
    _, lf = _run(OracleDecoder(OracleModel(d, w, kv="fp32"), 32), prompt, 5, forced)
    worst = max(_rel(a, b) for fa, fb in zip(lb, lf) for a, b in zip(fa, fb))
    assert 1e-5 < worst < 1e-2
