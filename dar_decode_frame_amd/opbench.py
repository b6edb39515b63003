"""Time single operations of the decode path through the C ABI (no model).

  python -m dar_decode_frame_amd.opbench gemm --wtype bf16 --rows 128 16 64 --shapes qkv wo w1 w2 --iters 50

gemm: dar_op_gemm_noalloc (the prefill / batched-decode MFMA GEMM: the hi/lo
split of the input rows, the K-split GEMM and, with more than one split, its
reduction) on the full-size matrices of one decoder layer (d 2560, 32/8 heads
of 128, SwiGLU 9728), `iters` back-to-back calls per shape on one stream,
timed with HIP events; the weights of consecutive calls rotate over eight
copies of the matrix so that no call finds its weights in the 256 MB
last-level cache. Prints one JSON line per (shape, rows). Under rocprofv3 the
GEMM kernel's own duration is in the kernel trace.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys

SHAPES = {  # (N, K) of one layer's projections at d 2560
    "qkv": (6144, 2560),
    "wo": (2560, 4096),
    "w1": (9728, 2560),
    "w2": (2560, 9728),
}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("op", choices=["gemm"])
    ap.add_argument("--wtype", default="bf16", choices=["bf16", "fp8", "int8", "int4"])
    ap.add_argument("--rows", type=int, nargs="+", default=[128])
    ap.add_argument("--shapes", nargs="+", default=list(SHAPES))
    ap.add_argument("--iters", type=int, default=50)
    ap.add_argument("--copies", type=int, default=8)
    args = ap.parse_args(argv)

    import torch

    from . import native as N

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    wt = N.WTYPES[args.wtype]
    gen = torch.Generator(device=dev).manual_seed(0)
    for name in args.shapes:
        n, k = SHAPES[name]
        ws, ss = [], []
        for _ in range(args.copies):
            w = (torch.randn(n, k, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
            if args.wtype == "bf16":
                ws.append(w)
                ss.append(None)
                continue
            if args.wtype == "int4":
                q = torch.empty(n, k // 2, dtype=torch.uint8, device=dev)
                s = torch.empty(n, k // 128, dtype=torch.float32, device=dev)
                fn = N.dar_quantize_int4_groups
            else:
                q = torch.empty(n, k, dtype=torch.uint8, device=dev)
                s = torch.empty(n, dtype=torch.float32, device=dev)
                fn = N.dar_quantize_fp8_rows if args.wtype == "fp8" else N.dar_quantize_int8_rows
            torch.cuda.synchronize()
            fn(ctypes.c_void_p(w.data_ptr()), n, k, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()), None)
            torch.cuda.synchronize()
            ws.append(q)
            ss.append(s)
            del w
        for m in args.rows:
            x = torch.randn(m, k, device=dev, generator=gen)
            y = torch.empty(m, n, device=dev)
            torch.cuda.synchronize()
            st = ctypes.c_void_p(stream.cuda_stream)

            def call(i):
                s = ss[i % args.copies]
                N.dar_op_gemm_noalloc(wt, ctypes.c_void_p(ws[i % args.copies].data_ptr()),
                                      ctypes.c_void_p(s.data_ptr()) if s is not None else None, n, k,
                                      ctypes.c_void_p(x.data_ptr()), m, ctypes.c_void_p(y.data_ptr()), st)

            for i in range(5):
                call(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.iters):
                call(i)
            e1.record(stream)
            stream.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / args.iters
            wbytes = ws[0].numel() * ws[0].element_size() + (ss[0].numel() * 4 if ss[0] is not None else 0)
            print(json.dumps({"op": "gemm", "wtype": args.wtype, "shape": name, "N": n, "K": k, "M": m,
                              "us_per_call": round(us, 2), "weight_tb_s": round(wbytes / us / 1e6, 3),
                              "tflop_s": round(2 * m * n * k / us / 1e6, 1)}), flush=True)
        del ws, ss
        torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
