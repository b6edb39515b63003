#!/usr/bin/env python3
"""Benchmark: batch-1 Dual-AR decode frames/s and achieved bandwidth on one MI355X.

Workload (default s2pro_dual_bf16): 36 slow layers + 4 fast layers x 9
residual codebooks, d 2560, 32/8 heads of 128, SwiGLU 9728, 4096-entry
codebooks, random-init N(0, 0.02) bf16 weights, prefill 128 random ids, then
decode frames at positions 128.. (the tuna-fish README's "prefill 128, decode
896" run to a 1024 context). A step is one decode frame: the fast AR of frame
i and the slow step of frame i+1 on two streams (eager launches; --graph
replays captured graphs instead). Inputs are resident in HBM before timing starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DTYPE_NAMES = {"bf16": "bf16", "fp8": "fp8_e4m3", "int8": "int8", "int4": "int4"}  # the weights' arithmetic type (activations fp32)
METRIC = "Dual-AR decode frames/s @batch1 + achieved HBM GB/s (% of ~8 TB/s peak)"
HBM_PEAK = 8.0e12
WEIGHT_KINDS = ("qkv", "wo", "w13", "w2", "head")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed frames (default: 896 at batch 1; a batched workload runs until its longest "
                         "sequence reaches max_len)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="s2pro_dual_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-frames", type=int, default=3)
    ap.add_argument("--graph", action="store_true", help="replay captured graphs instead of eager launches")
    ap.add_argument("--sample", action="store_true",
                    help="sample the codes instead of the argmax (stand-in settings, the pages give none: "
                         "temperature 0.8, top-k 50, top-p 0.9, repetition penalty 1.2 over 16 frames)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device to device once (a known-size reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from dar_decode_frame_amd import bytes_model as bm
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights

    if args.calibrate_copy > 0:
        # a device copy of known size, for scaling the profiler's HBM byte counters
        n = args.calibrate_copy * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy} MiB done")
        del src, dst
    if args.workload in synth.CODEC_WORKLOADS:
        return bench_codec(args, synth.CODEC_WORKLOADS[args.workload])
    wl = synth.WORKLOADS[args.workload]
    dims = wl.dims
    if wl.requests > 0:
        return bench_continuous(args, wl)
    if wl.batch != 1:
        return bench_batched(args, wl)
    max_steps = wl.max_len - wl.prefill_len
    if args.steps is None:
        args.steps = 896
    if args.steps > max_steps or args.steps < 1:
        raise SystemExit(f"--steps must be in [1, {max_steps}] for {wl.name}")
    dev = torch.device("cuda:0")

    t0 = time.time()
    host = synth.gen_weights(dims, wl.weight_seed)
    log(f"generated {len(host)} tensors in {time.time() - t0:.1f}s")
    t0 = time.time()
    weights = DeviceWeights(dims, host, wl.wtype, dev)
    log(f"uploaded{' and quantised' if wl.wtype != 'bf16' else ''} in {time.time() - t0:.1f}s")
    prompt = synth.gen_prompt(wl.prefill_len, dims.vocab_c0, wl.prompt_seed)
    sess = DarSession(dims, weights, wl.max_len, dev, graph=args.graph)
    set_sampling(sess, dims, wl, args)
    stream = sess.stream

    # warmup: prefill, W frames (captures the graph), then start over
    t0 = time.time()
    sess.prefill(prompt, want=False)
    stream.synchronize()
    for _ in range(args.warmup):
        sess.decode_frame(want=False)
    stream.synchronize()
    log(f"warmup ({args.warmup} frames) done in {time.time() - t0:.1f}s")
    sess.reset()
    ev_p0 = torch.cuda.Event(enable_timing=True)
    ev_p1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev_p0.record(stream)
    sess.prefill(prompt, want=False)
    with torch.cuda.stream(stream):
        ev_p1.record(stream)
    stream.synchronize()
    prefill_ms = ev_p0.elapsed_time(ev_p1)

    # timed region: K frames back to back, HIP events on the session stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # 64-frame windows at the start and the end of the run (shortest and longest KV)
    W64 = 64 if args.steps >= 128 else 0
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        if W64 and i == W64:
            ev_w[0].record(stream)
        if W64 and i == args.steps - W64:
            ev_w[1].record(stream)
        sess.decode_frame(want=False)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    windows = None
    if W64:
        windows = {}
        for name, t0_ev, t1_ev, first in (("first64", ev0, ev_w[0], 0), ("last64", ev_w[1], ev1, args.steps - W64)):
            wms = t0_ev.elapsed_time(t1_ev)
            wbytes = bm.run_bytes(dims, wl.wtype, wl.prefill_len + 1 + first, W64)
            windows[name] = {"kv_positions": [wl.prefill_len + 1 + first, wl.prefill_len + first + W64],
                             "frames_s": round(W64 * 1000.0 / wms, 2), "gb_s": round(wbytes / (wms / 1000.0) / 1e9, 1)}
    fps = args.steps * 1000.0 / ms
    t_first = wl.prefill_len + 1
    alg_bytes = bm.run_bytes(dims, wl.wtype, t_first, args.steps)
    gbs = alg_bytes / (ms / 1000.0)
    log(f"timed {args.steps} frames: {ms:.1f} ms, {fps:.1f} frames/s, {gbs / 1e9:.0f} GB/s")
    n_bad = sess.nonfinite()
    codes = sess.ring(wl.prefill_len - 1, args.steps + 1)

    # dominant kernel: the kind with the largest share of serialised frames
    # (both chains on one stream, every launch timed by a pair of HIP events
    # that the launch itself stamps at the kernel's start and end: the
    # kernels' own durations, as rocprofv3, which also serialises the streams,
    # reports them). Its launches are then also timed live on their own
    # streams over a second pass of the two-stream frames, where a launch
    # shares HBM with the other chain's kernels.
    roof = None
    if args.profile_frames > 0:
        sess.reset()
        sess.prefill(prompt, want=False)
        recs = []
        for _ in range(args.profile_frames):
            recs += sess.profile_frame()
        totals = {}
        for ms_k, kind, layer in recs:
            totals[kind] = totals.get(kind, 0.0) + ms_k
        # the weight-streaming kinds only: their bytes per launch are fixed
        # (attention's grow with the position, commits move a few KB)
        dom = max((k for k in totals if N.KIND_NAMES[k] in WEIGHT_KINDS), key=totals.get)
        share = {N.KIND_NAMES[k]: round(v / sum(totals.values()), 4)
                 for k, v in sorted(totals.items(), key=lambda kv: -kv[1])}
        # one-row launches only (the fast AR's first pass runs two rows)
        one_row = [ms_k for ms_k, kind, layer in recs if kind == dom and not (1000 <= layer < 2000)]
        avg_ms = sum(one_row) / len(one_row)
        sess.reset()
        sess.prefill(prompt, want=False)
        sess.time_kind(dom)
        for _ in range(args.steps):
            sess.decode_frame(want=False)
        live_ms, live_n = sess.kind_time()
        sess.time_kind(-1)
        name = N.KIND_NAMES[dom]
        per = per_launch_bytes(dims, wl.wtype, name)
        achieved = per / (avg_ms / 1000.0)
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                "traffic": measured_traffic(name, wl.name),
                "bytes_per_launch": per, "avg_launch_us": round(avg_ms * 1000, 2), "launches_timed": len(one_row),
                "overlapped_avg_launch_us": round(live_ms / live_n * 1000, 2) if live_n else None, "overlapped_launches": live_n,
                "launches_per_frame": len(recs) // args.profile_frames, "frame_time_share": share}
        rp = rocprof_launch_us(name, wl.name)
        roof["rocprof_avg_launch_us"] = rp
        roof["rocprof_frac"] = round(per / (rp * 1e-6) / HBM_PEAK, 4) if rp else None
        log(f"dominant kernel {name}: {avg_ms * 1000:.1f} us/launch serialised ({achieved / 1e9:.0f} GB/s), "
            + (f"{live_ms / live_n * 1000:.1f} us beside the other chain" if live_n else "no live timing (graph replay)")
            + f"; serialised-frame shares {share}")

    ref_read = reference_read(gbs)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dims, wl, host, prompt)

    out = {
        "metric": METRIC,
        "value": round(fps, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[wl.wtype],
        "data": "synthetic (seeded random-init weights and prompt ids)",
        "config": {"workload": wl.name, "batch": 1, "prefill": wl.prefill_len, "first_decode_position": wl.prefill_len,
                   "decode_frames": args.steps, "max_len": wl.max_len, "layers_slow": dims.n_layers_slow,
                   "layers_fast": dims.n_layers_fast, "residual_codebooks": dims.n_res,
                   "graph": args.graph, "sampling": SAMPLING if args.sample else None},
        "achieved_gb_s": round(gbs / 1e9, 1),
        "hbm_frac": round(gbs / HBM_PEAK, 4), "achieved_gib_s": round(gbs / bm.GIB, 1),
        "pages_formula": pages_formula(dims, wl, fps), "windows": windows,
        "alg_bytes_per_frame_avg": int(alg_bytes // args.steps),
        # dar_prefill runs the prompt blocks, the codebook-0 head and frame 0
        # (its codes are the call's output), so the blocks alone take about
        # one frame less
        "reference_read": ref_read,
        "prefill_ms": round(prefill_ms, 2), "prefill_blocks_ms_est": round(prefill_ms - ms / args.steps, 2),
        "prefill_tok_s_est": round(wl.prefill_len * 1000.0 / max(prefill_ms - ms / args.steps, 1e-6), 1),
        "nonfinite_logits": n_bad,
        "codes_checksum": int(np.asarray(codes, dtype=np.int64).sum()),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    sess.close()
    print(json.dumps(out), flush=True)


def bench_batched(args, wl):
    """Batched decode (the workload's sequences in lockstep, ragged prompts):
    aggregate frames/s over --steps lockstep steps (default: until the longest
    sequence reaches max_len), algorithmic bytes = the
    weights once per step + every sequence's KV reads, and the dominant
    launch kind of serialised steps against HBM and its MFMA rate."""
    import numpy as np
    import torch

    import synth
    from dar_decode_frame_amd import bytes_model as bm
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights

    dims, B = wl.dims, wl.batch
    dev = torch.device("cuda:0")
    lens, prompts = synth.gen_ragged_prompts(B, wl.prefill_len, wl.prefill_len_max, dims.vocab_c0, wl.prompt_seed,
                                            wl.length_seed)
    max_steps = wl.max_len - int(lens.max())
    steps = max_steps if args.steps is None else min(args.steps, max_steps)
    t0 = time.time()
    host = synth.gen_weights(dims, wl.weight_seed)
    weights = DeviceWeights(dims, host, wl.wtype, dev)
    if args.no_cpu_baseline:
        del host
    log(f"weights ready in {time.time() - t0:.1f}s; {B} prompts of {int(lens.min())}..{int(lens.max())} ids")
    sess = DarSession(dims, weights, wl.max_len, dev, graph=args.graph, batch=B)
    set_sampling(sess, dims, wl, args)
    stream = sess.stream
    sess.prefill(prompts, want=False)
    for _ in range(args.warmup):
        sess.decode_frame(want=False)
    stream.synchronize()
    sess.reset()
    ev_p0, ev_p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_p0.record(stream)
    sess.prefill(prompts, want=False)
    ev_p1.record(stream)
    stream.synchronize()
    prefill_ms = ev_p0.elapsed_time(ev_p1)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        sess.decode_frame(want=False)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    fps = B * steps * 1000.0 / ms
    # step i of sequence b attends T = lens[b] + 1 + i slow positions
    weights_b = bm.slow_weight_bytes(dims, wl.wtype) + dims.n_res * bm.fast_pass_bytes(dims, wl.wtype)
    kv = sum(bm.kv_bytes_per_position(dims) * (steps * (int(n) + 1) + steps * (steps - 1) // 2)
             + steps * bm.fast_kv_bytes(dims) for n in lens)
    alg_bytes = steps * weights_b + kv
    gbs = alg_bytes / (ms / 1000.0)
    log(f"timed {steps} steps x {B} sequences: {ms:.1f} ms, {fps:.1f} frames/s, {gbs / 1e9:.0f} GB/s")

    roof = None
    if args.profile_frames > 0:
        sess.reset()
        sess.prefill(prompts, want=False)
        recs = []
        for _ in range(args.profile_frames):
            recs += sess.profile_frame()
        totals = {}
        for ms_k, kind, layer in recs:
            totals[kind] = totals.get(kind, 0.0) + ms_k
        share = {N.KIND_NAMES[k]: round(v / sum(totals.values()), 4)
                 for k, v in sorted(totals.items(), key=lambda kv: -kv[1])}
        gemm_kinds = [k for k in sorted(totals, key=totals.get, reverse=True) if N.KIND_NAMES[k] in ("w13", "w2", "wo",
                                                                                                   "qkv")]
        dom = gemm_kinds[0]
        one_row = [m for m, kind, layer in recs if kind == dom and not (1000 <= layer < 2000)]
        avg_ms = sum(one_row) / len(one_row)
        name = N.KIND_NAMES[dom]
        # w13 launches are W1 and W3 separately here (one matrix each)
        per = per_launch_bytes(dims, wl.wtype, name) // (2 if name == "w13" else 1)
        flops = 2 * 2 * B * per / (2 if wl.wtype == "bf16" else 1)  # inputs as hi + lo bf16: two MFMA passes
        achieved = per / (avg_ms / 1000.0)
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4), "traffic": None, "bytes_per_launch": per,
                "avg_launch_us": round(avg_ms * 1000, 2), "launches_timed": len(one_row),
                "mfma_tflops": round(flops / (avg_ms / 1000.0) / 1e12, 1), "mfma_frac_bf16_dense": round(
                    flops / (avg_ms / 1000.0) / 2.5e15, 4),
                "launches_per_frame": len(recs) // args.profile_frames, "frame_time_share": share}
        log(f"dominant GEMM {name}: {avg_ms * 1000:.1f} us/launch, {achieved / 1e9:.0f} GB/s; shares {share}")
    n_bad = sess.nonfinite()
    sess.close()
    cpu = None
    if not args.no_cpu_baseline:
        del sess, weights
        torch.cuda.empty_cache()
        cpu = cpu_baseline_batched(dims, wl, host, lens, prompts)
        del host
    out = {
        "metric": METRIC, "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_NAMES[wl.wtype],
        "data": "synthetic (seeded random-init weights, ragged random prompts)",
        "config": {"workload": wl.name, "batch": B, "prompt_lengths": [int(n) for n in lens], "max_len": wl.max_len,
                   "layers_slow": dims.n_layers_slow, "layers_fast": dims.n_layers_fast,
                   "residual_codebooks": dims.n_res, "graph": args.graph,
                   "sampling": SAMPLING if args.sample else None},
        "achieved_gb_s": round(gbs / 1e9, 1), "hbm_frac": round(gbs / HBM_PEAK, 4),
        "alg_bytes_per_step_avg": int(alg_bytes // steps), "prefill_ms": round(prefill_ms, 2),
        "prefill_blocks_ms_est": round(prefill_ms - ms / steps, 2),
        "nonfinite_logits": n_bad, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_continuous(args, wl):
    """Continuous batching over the paged slow KV cache: wl.batch slots serve
    wl.requests requests in arrival order; a request joins (its prompt is
    prefilled) as soon as a slot is free, its frames come out of the following
    frame calls, and it leaves after its frame count. The timed region runs
    from the first admission to the last frame and includes the admissions'
    prefills. value = frames delivered / elapsed; algorithmic bytes count each
    frame call's weights once and every active request's slow KV reads."""
    import ctypes

    import numpy as np
    import torch

    import synth
    from dar_decode_frame_amd import bytes_model as bm
    from dar_decode_frame_amd import native as N
    from dar_decode_frame_amd.session import DarSession, DeviceWeights

    dims, S = wl.dims, wl.batch
    dev = torch.device("cuda:0")
    lens, nframes, prompts = synth.gen_requests(wl.requests, wl.prefill_len, wl.prefill_len_max, wl.frames_min,
                                                wl.decode_frames, dims.vocab_c0, wl.prompt_seed, wl.length_seed)
    t0 = time.time()
    host = synth.gen_weights(dims, wl.weight_seed)
    weights = DeviceWeights(dims, host, wl.wtype, dev)
    if args.no_cpu_baseline:
        del host
    log(f"weights ready in {time.time() - t0:.1f}s; {wl.requests} requests, prompts {int(lens.min())}..."
        f"{int(lens.max())} ids, {int(nframes.min())}..{int(nframes.max())} frames, {S} slots")
    sess = DarSession(dims, weights, wl.max_len, dev, batch=S, paging=(wl.page_len, wl.n_pages))
    stream, ctx = sess.stream, sess.ctx
    # every prompt resident on the device before timing
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    toks = torch.as_tensor(np.concatenate(prompts).astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    base = toks.data_ptr()

    def add(slot, r):
        N.dar_seq_add(ctx, slot, ctypes.c_void_p(base + 4 * int(offs[r])), int(lens[r]))

    # warmup: fill the slots, a few frames, empty them again
    for b in range(S):
        add(b, b)
    for _ in range(args.warmup):
        N.dar_decode_frame(ctx, None, None, None)
    for b in range(S):
        N.dar_seq_remove(ctx, b)
    stream.synchronize()

    kvp = bm.kv_bytes_per_position(dims)
    weights_b = bm.slow_weight_bytes(dims, wl.wtype) + dims.n_res * bm.fast_pass_bytes(dims, wl.wtype)
    queue = list(range(wl.requests))
    slot_req, left, pos = [None] * S, [0] * S, [0] * S
    calls = frames = active_sum = 0
    alg_bytes = 0
    min_free = sess.pages_free()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    while queue or any(r is not None for r in slot_req):
        for b in range(S):
            if slot_req[b] is None and queue:
                r = queue.pop(0)
                add(b, r)
                slot_req[b], left[b], pos[b] = r, int(nframes[r]), int(lens[r]) - 1
        min_free = min(min_free, N.dar_pages_free(ctx))
        N.dar_decode_frame(ctx, None, None, None)
        calls += 1
        alg_bytes += weights_b
        for b in range(S):
            if slot_req[b] is None:
                continue
            alg_bytes += kvp * (pos[b] + 2) + bm.fast_kv_bytes(dims)  # its slow step attends pos + 2 positions
            pos[b] += 1
            left[b] -= 1
            frames += 1
            active_sum += 1
            if left[b] == 0:
                N.dar_seq_remove(ctx, b)
                slot_req[b] = None
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    fps = frames * 1000.0 / ms
    gbs = alg_bytes / (ms / 1000.0)
    assert frames == int(nframes.sum())
    page_bytes = 2 * dims.n_layers_slow * dims.n_heads_kv * wl.page_len * dims.head_dim * 2
    log(f"timed {wl.requests} requests, {frames} frames in {calls} frame calls: {ms:.1f} ms, {fps:.1f} frames/s, "
        f"{gbs / 1e9:.0f} GB/s, mean {active_sum / calls:.1f} active slots, peak "
        f"{wl.n_pages - 1 - min_free} of {wl.n_pages - 1} pages")

    # dominant GEMM (W1 or W3, one matrix per launch) timed live over frames with every slot busy
    for b in range(S):
        add(b, b)
    sess.time_kind(3)
    for _ in range(32):
        N.dar_decode_frame(ctx, None, None, None)
    live_ms, live_n = sess.kind_time()
    sess.time_kind(-1)
    per = per_launch_bytes(dims, wl.wtype, "w13") // 2
    avg_ms = live_ms / live_n
    achieved = per / (avg_ms / 1000.0)
    roof = {"kernel": "w13", "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4), "traffic": None, "bytes_per_launch": per,
            "avg_launch_us": round(avg_ms * 1000, 2), "launches_timed": live_n,
            "note": "W1 and W3 GEMMs over the 16 slots' rows, timed live on their stream beside the other chain"}
    n_bad = sess.nonfinite()
    sess.close()
    cpu = None
    if not args.no_cpu_baseline:
        del sess, weights
        torch.cuda.empty_cache()
        cpu = cpu_baseline_batched(dims, wl, host, lens, prompts)
        del host
    out = {
        "metric": METRIC, "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1, "steps": calls,
        "warmup": args.warmup, "ms_per_step": round(ms / calls, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_NAMES[wl.wtype],
        "data": "synthetic (seeded random-init weights, random prompts, seeded request lengths)",
        "config": {"workload": wl.name, "slots": S, "requests": wl.requests,
                   "prompt_lengths": [int(lens.min()), int(lens.max())],
                   "frames_per_request": [int(nframes.min()), int(nframes.max())], "frames_total": frames,
                   "page_len": wl.page_len, "n_pages": wl.n_pages, "max_len": wl.max_len,
                   "layers_slow": dims.n_layers_slow, "layers_fast": dims.n_layers_fast,
                   "residual_codebooks": dims.n_res},
        "achieved_gb_s": round(gbs / 1e9, 1), "hbm_frac": round(gbs / HBM_PEAK, 4),
        "mean_active_slots": round(active_sum / calls, 2), "pages_peak": wl.n_pages - 1 - min_free,
        "kv_pool_bytes": wl.n_pages * page_bytes,
        "kv_bytes_lockstep_same_max_len": S * (wl.max_len // wl.page_len) * page_bytes,
        "nonfinite_logits": n_bad, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


CODEC_TAGS = {0: "rvq", 1: "in_conv", 2: "up", 3: "res_conv7", 4: "res_conv1", 5: "out_conv", 6: "res_unit"}
MFMA_BF16_PEAK = 2.5e15


def codec_launch_cost(d, frames, tag):
    """(FLOPs, bytes) one launch of a codec kind moves, averaged over the
    launches of the kind: the convolution's multiply-adds (2 per weight per
    output row per tap) and the activations it must read and write; weights
    counted once. Every convolution reads its operand, bf16(Snake(x)), which
    the layer before wrote: the input convolution and a block's last residual
    unit write only that, the transposed convolutions and the other units
    write it beside their fp32 rows (the residual stream, which the next
    residual add reads); an unfused unit also writes and reads its bf16 hidden
    rows, a one-launch unit keeps them on chip."""
    kind, blk = tag % 16, tag // 16
    w = d.widths
    U = len(d.dilations)  # residual units per block
    out_b = (6 * (U - 1) + 2) / U  # bytes per output element of a block's units: fp32 + operand, the last operand
    if kind == 0:
        return 0, frames * d.n_codebooks * d.latent_dim * 2 + frames * d.latent_dim * 2
    if kind == 1:
        return (2 * frames * w[0] * d.latent_dim * d.kernel,
                frames * d.latent_dim * 2 + frames * w[0] * 2 + w[0] * d.latent_dim * d.kernel * 2)
    rows_in = frames
    for s in d.rates[:blk]:
        rows_in *= s
    cin, cout, s = w[blk], w[blk + 1], d.rates[blk]
    rows = rows_in * s
    if kind == 2:
        return 2 * rows * cout * cin * 2, rows_in * cin * 2 + rows * cout * 6 + cin * cout * 2 * s * 2
    if kind == 3:
        return 2 * rows * cout * cout * d.kernel, rows * cout * 2 + rows * cout * 2 + cout * cout * d.kernel * 2
    if kind == 4:
        return 2 * rows * cout * cout, int(rows * cout * (2 + 4 + out_b)) + cout * cout * 2
    if kind == 6:
        return 2 * rows * cout * cout * (d.kernel + 1), int(rows * cout * (2 + 4 + out_b)) + cout * cout * (d.kernel + 1) * 2
    rows_out = frames * d.hop
    return 2 * rows_out * w[-1] * d.kernel, rows_out * w[-1] * 2 + rows_out * 4


def bench_codec(args, wl):
    """RVQ codec decode of one clip per step (codes resident in HBM, audio
    written to HBM): audio seconds decoded per second (x realtime) and the
    real-time factor; the dominant launch kind against bf16 MFMA peak."""
    import numpy as np
    import torch

    import synth
    from dar_decode_frame_amd.session import CodecSession

    d = wl.dims
    steps = args.steps if args.steps is not None else 20
    dev = torch.device("cuda:0")
    t0 = time.time()
    host = synth.gen_codec_weights(d, wl.weight_seed)
    codes = synth.gen_codes(wl.frames, d, wl.code_seed)
    sess = CodecSession(d, host, wl.frames, dev)
    sess.load_codes(codes)
    log(f"codec weights ready in {time.time() - t0:.1f}s; {wl.frames} frames -> {wl.frames * d.hop} samples")
    for _ in range(args.warmup):
        sess.decode(frames=wl.frames, want=False)
    sess.stream.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(sess.stream)
    for _ in range(steps):
        sess.decode(frames=wl.frames, want=False)
    ev1.record(sess.stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    audio_s = wl.frames * d.hop / d.sample_rate
    xrt = audio_s / (ms / 1000.0)
    log(f"timed {steps} decodes: {ms:.3f} ms each, {xrt:.0f}x realtime, RTF {ms / 1000.0 / audio_s:.2e}")
    audio = sess.decode(frames=wl.frames)
    flops = sum(codec_launch_cost(d, wl.frames, t)[0] for _, t in sess.profile(wl.frames))
    roof = None
    if args.profile_frames > 0:
        recs = []
        for _ in range(max(1, args.profile_frames)):
            recs += sess.profile(wl.frames)
        totals = {}
        for m, t in recs:
            totals[t] = totals.get(t, 0.0) + m
        dom = max((t for t in totals if t % 16 != 0), key=totals.get)
        times = [m for m, t in recs if t == dom]
        avg = sum(times) / len(times)
        f, b = codec_launch_cost(d, wl.frames, dom)
        # the kind's roofline: MFMA if its FLOPs per algorithmic byte exceed
        # the part's balance point (2.5 PFLOP/s / 8 TB/s = 312), else HBM
        mfma = f / b >= MFMA_BF16_PEAK / HBM_PEAK
        achieved = (f if mfma else b) / (avg / 1000.0)
        peak = MFMA_BF16_PEAK if mfma else HBM_PEAK
        share = {f"{CODEC_TAGS[t % 16]}{'' if t % 16 in (0, 1, 5) else t // 16}": round(v / sum(totals.values()), 4)
                 for t, v in sorted(totals.items(), key=lambda kv: -kv[1])}
        name = f"{CODEC_TAGS[dom % 16]}{'' if dom % 16 in (0, 1, 5) else dom // 16}"
        roof = {"kernel": name, "bound": "mfma" if mfma else "hbm",
                "achieved": round(achieved / (1e12 if mfma else 1e9), 1), "peak": peak / (1e12 if mfma else 1e9),
                "unit": "TFLOP/s" if mfma else "GB/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(name, wl.name, "dar_codec.hip"), "flops_per_launch": f,
                "bytes_per_launch": b, "avg_launch_us": round(avg * 1000, 2), "launches_timed": len(times),
                "tflop_s": round(f / (avg / 1000.0) / 1e12, 1), "hbm_gb_s": round(b / (avg / 1000.0) / 1e9, 1),
                "mfma_frac": round(f / (avg / 1000.0) / MFMA_BF16_PEAK, 4),
                "launches_per_step": len(recs) // max(1, args.profile_frames), "step_time_share": share}
        rp = rocprof_launch_us(name, wl.name, "dar_codec.hip")
        roof["rocprof_avg_launch_us"] = rp
        roof["rocprof_frac"] = round((f if mfma else b) / (rp * 1e-6) / peak, 4) if rp else None
        log(f"dominant kind {name}: {avg * 1000:.1f} us/launch, {f / (avg / 1000.0) / 1e12:.0f} TFLOP/s, "
            f"{b / (avg / 1000.0) / 1e9:.0f} GB/s; shares {share}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_codec(wl, host, codes)
    out = {
        "metric": "RVQ codec decode x realtime (audio seconds per second) @batch1",
        "value": round(xrt, 1),
        "unit": "x realtime",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init codec weights and codes)",
        "config": {"workload": wl.name, "batch": 1, "frames": wl.frames, "samples": wl.frames * d.hop,
                   "sample_rate": d.sample_rate, "codebooks": d.n_codebooks, "latent_dim": d.latent_dim,
                   "channels": d.channels, "rates": list(d.rates)},
        "rtf": round(ms / 1000.0 / audio_s, 8),
        "tflop_s": round(flops / (ms / 1000.0) / 1e12, 1),
        "flops_per_step": flops,
        "audio_checksum": round(float(np.abs(audio).sum()), 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    sess.close()
    print(json.dumps(out), flush=True)


def cpu_baseline_codec(wl, host, codes):
    """The codec oracle (NumPy fp64, bf16 activations) on this host's cores, on
    a window of the clip's frames sized to about 12 s of CPU work."""
    import numpy as np
    from oracle import CodecParams, codec_decode
    d = wl.dims
    threads = _blas_threads()
    P = CodecParams(d, host)
    n, t_dec = 4, 0.0
    while True:
        t0 = time.time()
        codec_decode(codes[:n], P, act="bf16")
        t_dec = time.time() - t0
        if t_dec > 6.0 or n >= wl.frames:
            break
        n = min(wl.frames, max(n + 1, int(n * 12.0 / max(t_dec, 1e-3))))
    audio_s = n * d.hop / d.sample_rate
    log(f"oracle: {n} frames ({audio_s:.3f} s of audio) in {t_dec:.1f}s on {threads} threads")
    return {"value": round(audio_s / t_dec, 4), "unit": "x realtime", "cores": threads, "kind": "oracle",
            "sample": f"{wl.name}: oracle (NumPy fp64, bf16 activations) decode of the first {n} frames "
                      f"({audio_s:.3f} s of audio) in {t_dec:.1f} s; weight conversion not timed",
            **_host_cpus()}


def pages_formula(dims, wl, fps):
    """The tuna-fish README's own decode-step bytes ("Inference estimation":
    parameters without embeddings, the fast AR once per pass, plus the static
    KV of max_length slow and R+1 fast positions, one byte count per element of
    the weight type) applied to this model, and the frame rate in its unit
    (GiB/s), the unit of the README's speed table."""
    from dar_decode_frame_amd import bytes_model as bm
    c = bm.param_counts(dims)
    p_slow = c["slow_layers"] + c["slow_final_norm"] + c["slow_head"]
    p_fast = bm.fast_params_wo_emb(dims) if dims.has_fast else 0
    passes = dims.n_res if dims.has_fast else 0
    elems = bm.pages_decode_elements(p_slow, p_fast, dims.n_layers_slow, dims.n_layers_fast,
                                     dims.n_heads_kv * dims.head_dim, wl.max_len, dims.n_res + 1, passes)
    per_elem = {"bf16": 2.0, "fp8": 1.0, "int8": 1.0, "int4": 0.5}[wl.wtype]
    step = elems * per_elem
    return {"bytes_per_step": int(step), "gib_s": round(fps * step / bm.GIB, 1)}


def reference_read(frame_bytes_per_s):
    """The GPU's own plain-read rate (dar_op_stream_read over 1 GiB: the
    fastest of its five launch shapes, five reads each, 16-byte non-temporal
    loads as the GEMVs use) and the frame's algorithmic byte rate as a
    fraction of it: context for hbm_frac, which is against the 8 TB/s
    datasheet figure."""
    import ctypes

    import torch

    from dar_decode_frame_amd import native as N
    buf = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    N.dar_op_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), 1, ctypes.c_void_p(sink.data_ptr()), None)
    ms = N.dar_op_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), 5, ctypes.c_void_p(sink.data_ptr()),
                              None)
    rate = buf.numel() / (ms * 1e-3)
    del buf, sink
    torch.cuda.empty_cache()
    log(f"reference read: {rate / 1e9:.0f} GB/s; the frame moves {frame_bytes_per_s / rate:.3f} of that")
    return {"kernel": "dar_op_stream_read", "bytes": 2 ** 30, "gb_s": round(rate / 1e9, 1),
            "frame_frac": round(frame_bytes_per_s / rate, 4)}


def measured_traffic(kind, workload, source="dar_kernels.hip"):
    """HBM bytes per launch of `kind` from the committed counter summary
    (profiles/hbm_traffic_<kind>_<workload>.md), or None when there is none or
    the kernel source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kind}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m_t or not m_h:
        return None
    src = os.path.join(ROOT, "dar_decode_frame_amd", "csrc", source)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_h.group(1):
        return None
    return int(m_t.group(1))


def rocprof_launch_us(kind, workload, source="dar_kernels.hip"):
    """The dominant kind's average launch duration in the committed rocprofv3
    kernel-trace summary of this workload's bench run (profiles/
    frame_kernels_<workload>.md: the kind's launches in the serialised frames,
    as the tracer timed them), or None when there is none or the kernel source
    has changed since the trace was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"frame_kernels_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_k = re.search(r"roofline_kind:\s*(\w+)", text)
    m_t = re.search(r"rocprof_avg_launch_us:\s*([0-9.]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not (m_k and m_t and m_h) or m_k.group(1) != kind:
        return None
    src = os.path.join(ROOT, "dar_decode_frame_amd", "csrc", source)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_h.group(1):
        return None
    return float(m_t.group(1))


SAMPLING = {"temperature": 0.8, "top_k": 50, "top_p": 0.9, "repetition_penalty": 1.2, "repetition_window": 16}


def set_sampling(sess, dims, wl, args):
    """With --sample: sampled codes, draws from a seeded table of uniforms."""
    if not args.sample:
        return
    import synth
    u = synth.gen_uniforms(wl.max_len, wl.batch, dims.n_res + 1, seed=3)
    sess.set_sampling(SAMPLING["temperature"], SAMPLING["top_k"], SAMPLING["top_p"],
                      SAMPLING["repetition_penalty"], SAMPLING["repetition_window"], u)


def per_launch_bytes(dims, wtype, kind):
    """Algorithmic bytes one single-row launch of `kind` reads (weights, their scales, norm gain)."""
    from dar_decode_frame_amd import bytes_model as bm
    d, F = dims.d_model, dims.ffn_dim

    def mat(rows, cols):
        return bm.matrix_bytes(wtype, rows, rows * cols)

    if kind == "w13":
        return mat(2 * F, d) + 2 * d
    if kind == "w2":
        return mat(d, F)
    if kind == "wo":
        return mat(d, dims.q_width)
    if kind == "qkv":
        return mat(dims.qkv_rows, d) + 2 * d
    if kind == "head":
        return dims.vocab_c0 * d * 2 + 2 * d
    raise ValueError(kind)


def cpu_baseline(dims, wl, host, prompt):
    """The oracle on this host's cores: prefill 128 then two decode frames; decode timed."""
    import numpy as np
    from oracle import OracleDecoder, OracleModel
    threads = _blas_threads()
    t0 = time.time()
    model = OracleModel(dims, host, wtype=wl.wtype)
    t_build = time.time() - t0
    dec = OracleDecoder(model, wl.max_len)
    t0 = time.time()
    dec.prefill(prompt)
    t_prefill = time.time() - t0
    # decode frames until about 12 s of CPU work (at least 2), within the capacity
    budget_s, frames = 12.0, 0
    t0 = time.time()
    while frames < 2 or (time.time() - t0 < budget_s and dec.pos < wl.max_len):
        dec.decode_frame()
        frames += 1
    t_dec = time.time() - t0
    log(f"oracle: build {t_build:.1f}s, prefill {t_prefill:.1f}s, {frames} frames {t_dec:.1f}s on {threads} threads")
    # the same decode on one BLAS thread, a shorter sample (about 6 s)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            f1, t1 = 0, time.time()
            while dec.pos < wl.max_len and (f1 < 1 or time.time() - t1 < 6.0):
                dec.decode_frame()
                f1 += 1
            one = round(f1 / (time.time() - t1), 4) if f1 else None
        log(f"oracle on one thread: {f1} frames, {one} frames/s")
    except ImportError:
        pass
    del model, dec
    return {"value": round(frames / t_dec, 4), "unit": "frames/s", "cores": threads, "kind": "oracle",
            "value_one_thread": one,
            "sample": f"{wl.name}: oracle (NumPy fp32) prefill {wl.prefill_len} as one causal block, then "
                      f"{frames} decode frames at positions {wl.prefill_len}..{wl.prefill_len + frames - 1} timed "
                      f"({t_dec:.1f} s, budget about 12 s); weight conversion {t_build:.1f} s and "
                      f"prefill {t_prefill:.1f} s not timed",
            **_host_cpus()}


def cpu_baseline_batched(dims, wl, host, lens, prompts):
    """The oracle on this host's cores for a batched workload: the oracle
    decodes one sequence at a time, so a sample of two of the batch's own
    sequences (prefill, then frames alternating between them until about 12 s
    of decode) gives its aggregate frames/s."""
    from oracle import OracleDecoder, OracleModel
    threads = _blas_threads()
    t0 = time.time()
    model = OracleModel(dims, host, wtype=wl.wtype)
    t_build = time.time() - t0
    picks = [0, 1]
    decs = []
    t0 = time.time()
    for b in picks:
        d = OracleDecoder(model, wl.max_len)
        d.prefill(prompts[b])
        decs.append(d)
    t_prefill = time.time() - t0
    budget_s, frames = 12.0, 0
    t0 = time.time()
    while frames < 2 or time.time() - t0 < budget_s:
        decs[frames % 2].decode_frame()
        frames += 1
    t_dec = time.time() - t0
    log(f"oracle: build {t_build:.1f}s, prefill {t_prefill:.1f}s, {frames} frames {t_dec:.1f}s on {threads} threads")
    del model, decs
    return {"value": round(frames / t_dec, 4), "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"{wl.name}: oracle (NumPy fp32), sequences {picks} of the batch (prompts of "
                      f"{[int(lens[b]) for b in picks]} ids) prefilled, then {frames} decode frames alternating "
                      f"between them timed ({t_dec:.1f} s, budget about 12 s; the oracle decodes one sequence at a "
                      f"time, so this is its aggregate rate); weight conversion {t_build:.1f} s and prefill "
                      f"{t_prefill:.1f} s not timed",
            **_host_cpus()}


def _blas_threads():
    """Threads the oracle's BLAS calls actually run on (the `cores` it used)."""
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 0) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        return os.cpu_count()


def _host_cpus():
    """The host's CPU model, its logical CPU count and the CPUs this process may run on."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": _cpu_model(), "host_cpu_count": os.cpu_count(), "usable_cpus": usable}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
