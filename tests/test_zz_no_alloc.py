"""sharq_forward_noalloc (the allocation-free variant of sharq_forward, for callers that
cannot allocate device memory) against sharq_forward, called through the C ABI: the
same payload bytes and outputs on two calls in a row, the second with a smaller input,
for both formats.  The variant's scratch is the library's fixed per-device array."""
import ctypes

import numpy as np
import pytest
import torch

from activation_sparsity_fp4_sharq_amd import sharq
from activation_sparsity_fp4_sharq_amd.workloads import make_shape

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _bytes(p):
    """The payload bytes a call writes (the tensor scale only for NVFP4: MXFP4 never writes it)."""
    out = [p.codes.cpu().numpy(), p.scales.cpu().numpy()]
    if p.fmt == sharq.NVFP4:
        out.append(p.tensor_scale[:1].cpu().numpy())
    return out


def _noalloc(x, weight, n, m, bb, rr, y, out_dtype):
    sb, sr, sw = bb.struct(), rr.struct(), weight.struct()
    M, K = x.shape
    return sharq.lib().sharq_forward_noalloc(
        ctypes.c_void_p(x.data_ptr()), M, K, x.stride(0), n, m, weight.fmt, ctypes.byref(sb), ctypes.byref(sr),
        ctypes.byref(sw), weight.rows, ctypes.c_void_p(y.data_ptr()), y.stride(0), out_dtype,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("fmt", [sharq.MXFP4, sharq.NVFP4], ids=["mx", "nv"])
@pytest.mark.parametrize("out_dtype", [sharq.OUT_FP32, sharq.OUT_BF16], ids=["fp32", "bf16"])
def test_noalloc_forward_matches_forward_on_two_calls(fmt, out_dtype):
    N, K = 384, 1024
    wb = make_shape(1, N, K, seed=11)[1]
    weight = sharq.quantize(to_dev(wb), fmt)
    for M, seed in ((700, 21), (90, 22)):  # the second call is smaller
        print(f"[noalloc] fmt={fmt} out={out_dtype} M={M} N={N} K={K}", flush=True)
        xb, _ = make_shape(M, N, K, seed=seed, dist="laplace", token_sigma=0.4)
        x = to_dev(xb)
        y_ref, (b_ref, r_ref) = sharq.forward(x, weight, 2, 4, out_dtype=out_dtype)
        bb = sharq.Payload.empty(M, K, fmt, DEV, weight.layout)
        rr = sharq.Payload.empty(M, K, fmt, DEV, weight.layout)
        y = torch.empty_like(y_ref)
        assert _noalloc(x, weight, 2, 4, bb, rr, y, out_dtype) == 0
        torch.cuda.synchronize()
        for got, want in zip(_bytes(bb) + _bytes(rr), _bytes(b_ref) + _bytes(r_ref)):
            assert np.array_equal(got, want)
        assert torch.equal(y.view(torch.int32 if out_dtype == sharq.OUT_FP32 else torch.int16),
                           y_ref.view(torch.int32 if out_dtype == sharq.OUT_FP32 else torch.int16))


def test_noalloc_binding_and_errors():
    print("[noalloc] binding / errors", flush=True)
    N, K, M = 128, 256, 40
    xb, wb = make_shape(M, N, K, seed=5)
    weight = sharq.quantize(to_dev(wb), sharq.NVFP4)
    y, (bb, rr) = sharq.forward_noalloc(to_dev(xb), weight, 4, 8, out_dtype=sharq.OUT_FP32)
    y_ref, _ = sharq.forward(to_dev(xb), weight, 4, 8, out_dtype=sharq.OUT_FP32)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    # invalid arguments are rejected before anything is enqueued
    x = to_dev(xb)
    assert _noalloc(x, weight, 3, 4, bb, rr, y, sharq.OUT_FP32) == 3  # SHARQ_E_PATTERN
