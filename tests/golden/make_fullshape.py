#!/usr/bin/env python3
"""Write the full-shape oracle references used by tests/test_gpu_fullshape.py.

Calls only oracle/ and synth/ (the CPU oracle at the benchmark's full shapes:
36 + 4 layers, d 2560, 32/8 heads of 128, SwiGLU 9728, 4096-entry codebooks).
For each workload it records two runs on the seeded weights and prompt:

- early: prefill 128 + 9 decode frames, teacher-forced with the oracle's own
  greedy frames (positions 127..136);
- late: frames forced with seeded random codes up to position 1007, where the
  oracle runs the prompt and the forced codebook-0 ids as one causal block and
  records the last frame only.

Per (frame, codebook) logit vector it stores the oracle's argmax and its
top-1 - top-2 margin (fullshape_<workload>.json) and the whole fp32 logit
vector (fullshape_<workload>.npz: "early" [frames][1 + n_res][4096], "late"
[1 + n_res][4096]). Slow to run (the fp8 oracle quantises 4 billion weights in
NumPy: minutes); run from the repository root:
  python3 tests/golden/make_fullshape.py [workload ...]
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import OracleDecoder, OracleModel  # noqa: E402

WORKLOADS = ["s2pro_slow_bf16", "s2pro_dual_bf16", "s2pro_dual_fp8", "s2pro_dual_int8", "s2pro_dual_int4"]
EARLY_FRAMES = 9
LATE_LAST_POS = 1007          # slow position of the late frame
FORCE_SEED = 4242


def random_frames(dims, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        c0 = rng.integers(dims.vocab_c0)
        res = rng.integers(0, dims.vocab_res, dims.n_res) if dims.n_res else np.zeros(0, np.int64)
        out.append([int(c0)] + [int(r) for r in res])
    return out


def record(frame, dims):
    """Per codebook: the oracle's code and top-1 - top-2 margin; and the logit
    vectors [1 + n_res][vmax] in fp32 (entries past a codebook's size zero)."""
    codes, logits = frame
    vmax = max(dims.vocab_c0, dims.vocab_res if dims.n_res else 0)
    vecs, full = [], np.zeros((dims.n_res + 1, vmax), dtype=np.float32)
    for k in range(dims.n_res + 1):
        V = dims.vocab_c0 if k == 0 else dims.vocab_res
        lg = np.asarray(logits[k][:V], dtype=np.float64)
        order = np.argsort(lg)
        vecs.append({"code": int(codes[k]), "margin": float(lg[order[-1]] - lg[order[-2]])})
        full[k, :V] = lg
    return vecs, full


def main(names):
    out_dir = os.path.dirname(os.path.abspath(__file__))
    for name in names:
        wl = synth.WORKLOADS[name]
        dims = wl.dims
        t0 = time.time()
        host = synth.gen_weights(dims, wl.weight_seed)
        model = OracleModel(dims, host, wtype=wl.wtype, drop_source=True)
        del host
        print(f"{name}: oracle built in {time.time() - t0:.0f} s", flush=True)
        prompt = synth.gen_prompt(wl.prefill_len, dims.vocab_c0, wl.prompt_seed)

        # early frames, forced with the oracle's own greedy frames
        dec = OracleDecoder(model, wl.max_len)
        frames = [dec.prefill(prompt)]
        for _ in range(EARLY_FRAMES):
            frames.append(dec.decode_frame())
        recs = [record(f, dims) for f in frames]
        early = {"forced": [[int(c) for c in f[0]] for f in frames], "frames": [r[0] for r in recs]}

        # late frame: forced random frames 0..K, frame K sits at position n - 1 + K
        K = LATE_LAST_POS - (wl.prefill_len - 1)
        forced = random_frames(dims, K + 1, FORCE_SEED)
        dec = OracleDecoder(model, wl.max_len)
        tokens = np.concatenate([prompt, np.array([f[0] for f in forced[:K]], dtype=prompt.dtype)])
        last = dec.prefill(tokens, forced=np.array(forced[K], dtype=np.int32))
        late_vecs, late_full = record(last, dims)
        late = {"force_seed": FORCE_SEED, "frames_forced": K + 1, "position": LATE_LAST_POS, "frame": late_vecs}
        doc = {"workload": name, "source": "tests/golden/make_fullshape.py (CPU oracle, oracle/model.py)",
               "weight_seed": wl.weight_seed, "prompt_seed": wl.prompt_seed, "prefill": wl.prefill_len,
               "max_len": wl.max_len, "early": early, "late": late}
        with open(os.path.join(out_dir, f"fullshape_{name}.json"), "w") as f:
            json.dump(doc, f, separators=(",", ":"))
        np.savez_compressed(os.path.join(out_dir, f"fullshape_{name}.npz"),
                            early=np.stack([r[1] for r in recs]), late=late_full)
        print(f"{name}: done in {time.time() - t0:.0f} s", flush=True)
        del model, dec


if __name__ == "__main__":
    # optional: the workloads to (re)write, default all
    main(sys.argv[1:] or WORKLOADS)
