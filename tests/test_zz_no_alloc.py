"""dar_op_gemm_noalloc, the GEMM entry point that allocates nothing (for
callers that cannot call hipMalloc: graph capture, serving loops), against the
allocating dar_op_gemm on the same inputs, on two calls in a row (the second
smaller), plus an fp64 reference of the product. Run alone or after the
other GPU tests."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("wtype", ["bf16", "fp8"])
def test_noalloc_gemm_equals_allocating_gemm_on_two_calls(wtype):
    import torch
    from dar_decode_frame_amd import native as N
    r = np.random.default_rng(11)
    wt = N.WTYPES[wtype]
    # first call: M 128 x N 9728 x K 2560 needs more partial sums than the
    # static array keeps beside the input halves (fewer K splits); second: smaller
    for M, Nn, K in [(128, 9728, 2560), (7, 2560, 1024)]:
        Wb = synth.f32_to_bf16_bits(r.standard_normal((Nn, K)).astype(np.float32) * 0.02)
        x = r.standard_normal((M, K)).astype(np.float32)
        Wd = torch.from_numpy(Wb.view(np.int16)).cuda()
        xd = torch.from_numpy(x).cuda()
        scale = None
        if wtype == "fp8":
            q = torch.empty(Nn, K, dtype=torch.uint8, device="cuda")
            scale = torch.empty(Nn, dtype=torch.float32, device="cuda")
            torch.cuda.synchronize()
            N.dar_quantize_fp8_rows(_p(Wd), Nn, K, _p(q), _p(scale), None)
            torch.cuda.synchronize()
            Wd = q
        y0 = torch.zeros(M, Nn, dtype=torch.float32, device="cuda")
        y1 = torch.full((M, Nn), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        sp = _p(scale) if scale is not None else None
        N.dar_op_gemm(wt, _p(Wd), sp, Nn, K, _p(xd), M, _p(y0), None)
        N.dar_op_gemm_noalloc(wt, _p(Wd), sp, Nn, K, _p(xd), M, _p(y1), None)
        torch.cuda.synchronize()
        a, b = y0.cpu().numpy().astype(np.float64), y1.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(b))
        # the weights each side multiplies, widened: bf16 values, or codes x row scale
        if wtype == "bf16":
            Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        else:
            codes = Wd.cpu().numpy()
            from oracle import e4m3_decode
            Wf = e4m3_decode(codes).astype(np.float64) * scale.cpu().numpy().astype(np.float64)[:, None]
        ref = x.astype(np.float64) @ Wf.T
        S = np.abs(x).astype(np.float64) @ np.abs(Wf).T
        assert np.all(np.abs(b - a) <= 2e-5 * S), np.max(np.abs(b - a) / S)
        assert np.all(np.abs(b - ref) <= 1e-5 * S), np.max(np.abs(b - ref) / S)
