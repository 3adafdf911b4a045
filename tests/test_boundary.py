"""The C ABI boundary on the CPU: the library loads, exports every function that
include/sharq.h declares, and rejects every invalid argument with its status before
touching the GPU (validation runs first, so these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

from activation_sparsity_fp4_sharq_amd import sharq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sharq.h")

OK, E_NULL, E_SHAPE, E_PATTERN, E_FORMAT, E_ALIGN, E_WORKSPACE, E_LAUNCH, E_DEVICE = range(9)
A = 0x10000  # a 16-byte aligned fake device address: never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sharq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert {"sharq_prep", "sharq_linear", "sharq_quantize", "sharq_forward"} <= set(names)
    L = sharq.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in sharq.h but not exported"
    assert set(names) == set(sharq.SYMBOLS)


def test_version_and_status_strings():
    L = sharq.lib()
    assert L.sharq_abi_version() == 12
    for s in range(9):
        assert L.sharq_status_str(s)
    assert L.sharq_status_str(99) == b"unknown status"


def test_workspace_sizes():
    L = sharq.lib()
    assert L.sharq_prep_workspace_bytes(4096, 4096, sharq.MXFP4) == 0
    assert L.sharq_prep_workspace_bytes(4096, 4096, sharq.NVFP4) >= 8
    assert L.sharq_linear_workspace_bytes(0, 10, 32, sharq.MXFP4) == 0
    assert L.sharq_linear_workspace_bytes(2048, 4096, 14336, sharq.MXFP4) == 0  # the split is optional


def test_split_workspace_sizes():
    """K splits for tiled MXFP4 shapes with fewer 256x256 tiles than 256 compute units:
    as many splits as fill them, at most 4, each with at least 16 K-steps of 128."""
    L = sharq.lib()
    f = L.sharq_linear_split_workspace_bytes
    assert f(2048, 4096, 14336, sharq.MXFP4) == 2 * 2048 * 4096 * 4  # 128 tiles, 112 steps
    assert f(600, 512, 8192, sharq.MXFP4) == 4 * 600 * 512 * 4      # 6 tiles: capped at 4
    assert f(300, 1000, 6144, sharq.MXFP4) == 3 * 300 * 1000 * 4    # 48 steps: 3 of 16
    assert f(4096, 4096, 4096, sharq.MXFP4) == 0                     # 256 tiles fill the part
    assert f(2048, 4096, 2048, sharq.MXFP4) == 0                     # 16 steps: one split
    assert f(32, 4096, 14336, sharq.MXFP4) == 0                      # the small-M kernel
    assert f(2048, 4096, 14336, sharq.NVFP4) == 0
    assert f(0, 4096, 14336, sharq.MXFP4) == 0 and f(64, 0, 4096, sharq.MXFP4) == 0


def fp4(codes=A, scales=A, ts=A, layout=0, reserved=0):
    return sharq.SharqFp4(codes, scales, ts, layout, reserved)


def prep(x=A, M=4, K=64, ldx=64, n=2, m=4, fmt=0, bb=None, rr=None, mask=None, ws=None, wsb=0):
    bb = bb if bb is not None else fp4()
    rr = rr if rr is not None else fp4()
    return sharq.lib().sharq_prep(x, M, K, ldx, n, m, fmt, ctypes.byref(bb), ctypes.byref(rr), mask, ws, wsb,
                                  None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), E_NULL),
    (dict(K=48), E_SHAPE),                 # not a multiple of 32 (MXFP4)
    (dict(K=0), E_SHAPE),
    (dict(M=-1), E_SHAPE),
    (dict(ldx=32), E_SHAPE),               # ldx < K
    (dict(n=3, m=4), E_PATTERN),
    (dict(n=2, m=8), E_PATTERN),
    (dict(fmt=7), E_FORMAT),
    (dict(x=A + 2), E_ALIGN),
    (dict(ldx=68), E_ALIGN),               # row starts not 16-byte aligned
    (dict(bb=fp4(codes=None)), E_NULL),
    (dict(rr=fp4(scales=A + 4)), E_ALIGN),
    (dict(mask=A + 1), E_ALIGN),
    (dict(fmt=1, bb=fp4(ts=None)), E_NULL),  # NVFP4 needs tensor scales
    (dict(fmt=1), E_WORKSPACE),              # NVFP4 needs workspace
    (dict(bb=fp4(layout=2)), E_FORMAT),       # unknown layout
    (dict(bb=fp4(reserved=1)), E_FORMAT),     # reserved field must be 0
    (dict(fmt=1, bb=fp4(layout=1), rr=fp4(layout=1)), E_FORMAT),  # tiled is MXFP4 only
    (dict(bb=fp4(layout=1)), E_FORMAT),       # backbone and residual layouts differ
])
def test_prep_rejects(kwargs, status):
    assert prep(**kwargs) == status


def test_prep_nvfp4_accepts_k16_shape_check():
    # K = 48 is valid for NVFP4 (multiple of 16); fails later only on the workspace
    assert prep(K=48, ldx=48, fmt=1) == E_WORKSPACE


def linear(M=4, N=8, K=64, fmt=0, y=A, ldy=8, out=0, bb=None, rr=None, w=None, ws=None, wsb=0):
    bb = bb if bb is not None else fp4()
    rr = rr if rr is not None else fp4()
    w = w if w is not None else fp4()
    return sharq.lib().sharq_linear(ctypes.byref(bb), ctypes.byref(rr), M, ctypes.byref(w), N, K, fmt, y, ldy,
                                    out, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(y=None), E_NULL),
    (dict(N=0), E_SHAPE),
    (dict(K=40), E_SHAPE),
    (dict(ldy=4), E_SHAPE),
    (dict(M=-2), E_SHAPE),
    (dict(fmt=3), E_FORMAT),
    (dict(out=5), E_FORMAT),
    (dict(y=A + 1), E_ALIGN),
    (dict(y=A + 2, out=1), E_ALIGN),
    (dict(w=fp4(codes=A + 8)), E_ALIGN),
    (dict(bb=fp4(scales=None)), E_NULL),
    (dict(fmt=1, w=fp4(ts=None)), E_NULL),
    (dict(w=fp4(layout=1)), E_FORMAT),        # mixed layouts
])
def test_linear_rejects(kwargs, status):
    assert linear(**kwargs) == status


def linear_dense(M=4, N=8, K=64, fmt=0, y=A, ldy=8, out=0, a=None, w=None, ws=None, wsb=0):
    a = a if a is not None else fp4()
    w = w if w is not None else fp4()
    return sharq.lib().sharq_linear_dense(ctypes.byref(a), M, ctypes.byref(w), N, K, fmt, y, ldy, out, ws, wsb,
                                          None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(y=None), E_NULL),
    (dict(N=0), E_SHAPE),
    (dict(K=40), E_SHAPE),
    (dict(K=40, fmt=1), E_SHAPE),             # not a multiple of 16 (NVFP4)
    (dict(ldy=4), E_SHAPE),
    (dict(M=-1), E_SHAPE),
    (dict(fmt=2), E_FORMAT),
    (dict(out=2), E_FORMAT),
    (dict(y=A + 1), E_ALIGN),
    (dict(a=fp4(codes=None)), E_NULL),
    (dict(a=fp4(scales=A + 2)), E_ALIGN),
    (dict(fmt=1, a=fp4(ts=None)), E_NULL),    # NVFP4 needs the activation's tensor scale
    (dict(a=fp4(layout=1)), E_FORMAT),        # activation and weight layouts differ
])
def test_linear_dense_rejects(kwargs, status):
    assert linear_dense(**kwargs) == status


def test_tiled_gemm_k_limit():
    """Tiled payloads: the pipelined GEMM addresses a row tile's K range with 32-bit
    offsets, so K above 2^27 is rejected before anything runs (row-major payloads keep the
    general 2^30 limit); K = 2^27 passes every shape check."""
    import torch
    t = dict(bb=fp4(layout=1), rr=fp4(layout=1), w=fp4(layout=1))
    assert linear(K=(1 << 27) + 32, **t) == E_SHAPE
    assert linear_dense(K=(1 << 27) + 32, a=fp4(layout=1), w=fp4(layout=1)) == E_SHAPE
    L = sharq.lib()
    bb, rr, w = fp4(layout=1), fp4(layout=1), fp4(layout=1)
    assert L.sharq_forward(A, 4, (1 << 27) + 32, (1 << 27) + 32, 2, 4, 0, ctypes.byref(bb), ctypes.byref(rr),
                           ctypes.byref(w), 8, A, 8, 0, None, 0, None) == E_SHAPE
    if not torch.cuda.is_available():
        assert linear(K=1 << 27, **t) == E_DEVICE
        assert linear(K=(1 << 27) + 32) == E_DEVICE  # row-major: past every shape check


def test_linear_null_backbone_is_rejected():
    rr, w = fp4(), fp4()
    assert sharq.lib().sharq_linear(None, ctypes.byref(rr), 4, ctypes.byref(w), 8, 64, 0, A, 8, 0, None, 0,
                                    None) == E_NULL


def test_prep_ablation_rejects():
    L = sharq.lib()
    bb, rr = fp4(), fp4()

    def call(variant=1, fmt=0, n=2, m=4, x=A, K=64, ws=None, wsb=0):
        return L.sharq_prep_ablation(x, 4, K, K, n, m, fmt, variant, ctypes.byref(bb), ctypes.byref(rr), None, ws,
                                     wsb, None)
    assert call(variant=0) == E_FORMAT     # the method itself is sharq_prep
    assert call(variant=4) == E_FORMAT
    assert call(n=3) == E_PATTERN
    assert call(x=None) == E_NULL
    assert call(K=48) == E_SHAPE
    assert call(fmt=1) == E_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        for v in (1, 2, 3):
            assert call(variant=v) == E_DEVICE


def test_prep_swiglu_rejects():
    L = sharq.lib()
    bb, rr = fp4(), fp4()

    def call(x=A, M=4, I=64, ld=128, n=2, m=4, fmt=0, ws=None, wsb=0):
        return L.sharq_prep_swiglu(x, M, I, ld, n, m, fmt, ctypes.byref(bb), ctypes.byref(rr), None, ws, wsb, None)
    assert call(ld=120) == E_SHAPE        # ld < 2I
    assert call(I=48) == E_SHAPE          # not a multiple of 32 (MXFP4)
    assert call(x=None) == E_NULL
    assert call(ld=132) == E_ALIGN        # rows not 16-byte aligned
    assert call(m=8, n=2) == E_PATTERN
    assert call(fmt=1) == E_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert call() == E_DEVICE


def test_dequantize_rejects():
    L = sharq.lib()
    p = fp4()
    assert L.sharq_dequantize(ctypes.byref(p), 4, 64, 0, None, 64, None) == E_NULL
    assert L.sharq_dequantize(ctypes.byref(p), 4, 48, 0, A, 64, None) == E_SHAPE
    assert L.sharq_dequantize(ctypes.byref(p), 4, 64, 0, A, 32, None) == E_SHAPE    # ldo < K
    assert L.sharq_dequantize(ctypes.byref(p), 4, 64, 0, A + 2, 64, None) == E_ALIGN
    assert L.sharq_dequantize(ctypes.byref(p), 4, 64, 3, A, 64, None) == E_FORMAT
    q = fp4(layout=1)
    assert L.sharq_dequantize(ctypes.byref(q), 4, 64, 1, A, 64, None) == E_FORMAT  # tiled NVFP4


def test_clock_probe_rejects():
    L = sharq.lib()
    assert L.sharq_clock_probe(100, None, None) == E_NULL
    assert L.sharq_clock_probe(0, A, None) == E_SHAPE
    assert L.sharq_clock_probe(100, A + 4, None) == E_ALIGN


def test_quantize_rejects():
    L = sharq.lib()
    out = fp4()
    assert L.sharq_quantize(None, 4, 64, 64, 0, ctypes.byref(out), None, 0, None) == E_NULL
    assert L.sharq_quantize(A, 4, 60, 64, 0, ctypes.byref(out), None, 0, None) == E_SHAPE
    assert L.sharq_quantize(A, 4, 64, 64, 1, ctypes.byref(out), None, 0, None) == E_WORKSPACE
    assert L.sharq_quantize(A, 4, 64, 64, 1, ctypes.byref(out), A + 8, 1 << 20, None) == E_ALIGN


def test_forward_rejects_before_launch():
    L = sharq.lib()
    bb, rr, w = fp4(), fp4(), fp4()
    args = dict(x=A, M=4, K=64, ldx=64, n=2, m=4, fmt=0, N=8, y=A, ldy=8, out=0)

    def call(**kw):
        a = {**args, **kw}
        return L.sharq_forward(a["x"], a["M"], a["K"], a["ldx"], a["n"], a["m"], a["fmt"], ctypes.byref(bb),
                               ctypes.byref(rr), ctypes.byref(w), a["N"], a["y"], a["ldy"], a["out"], None, 0,
                               None)
    assert call(ldy=4) == E_SHAPE        # the linear half is checked before the prep runs
    assert call(out=9) == E_FORMAT
    assert call(n=1) == E_PATTERN
    assert call(y=None) == E_NULL


def test_valid_call_without_gfx950_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert prep() == E_DEVICE
    assert linear() == E_DEVICE
    assert linear_dense() == E_DEVICE


def test_payload_bytes():
    L = sharq.lib()
    c, sc = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.sharq_payload_bytes(100, 96, 0, 0, ctypes.byref(c), ctypes.byref(sc)) == 100 * 48 + 100 * 3
    assert (c.value, sc.value) == (4800, 300)
    # tiled pads rows to 32 and K to 128
    assert L.sharq_payload_bytes(100, 96, 0, 1, ctypes.byref(c), ctypes.byref(sc)) == 128 * 64 + 128 * 4
    assert (c.value, sc.value) == (128 * 64, 128 * 4)
    assert L.sharq_payload_bytes(10, 64, 1, 1, None, None) == 0      # tiled NVFP4 does not exist
    assert L.sharq_payload_bytes(10, 48, 0, 0, None, None) == 0      # K not a multiple of 32
    assert L.sharq_payload_bytes(10, 48, 1, 0, None, None) == 10 * 24 + 10 * 3


def test_convert_rejects():
    L = sharq.lib()
    a, b = fp4(), fp4(layout=1)
    assert L.sharq_convert_layout(ctypes.byref(a), ctypes.byref(b), 4, 64, 1, None) == E_FORMAT
    assert L.sharq_convert_layout(ctypes.byref(a), ctypes.byref(b), 4, 48, 0, None) == E_SHAPE
    assert L.sharq_convert_layout(ctypes.byref(a), ctypes.byref(fp4(codes=None)), 4, 64, 0, None) == E_NULL


def prep_norm(x=A, M=4, K=64, ldx=64, gamma=A, eps=1e-6, n=2, m=4, fmt=0, bb=None, rr=None, mask=None, ws=A,
              wsb=1 << 20):
    bb = bb if bb is not None else fp4()
    rr = rr if rr is not None else fp4()
    return sharq.lib().sharq_prep_rmsnorm(x, M, K, ldx, gamma, eps, n, m, fmt, ctypes.byref(bb), ctypes.byref(rr),
                                          mask, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(gamma=None), E_NULL),
    (dict(gamma=A + 8), E_ALIGN),
    (dict(eps=-1.0), E_SHAPE),
    (dict(eps=float("nan")), E_SHAPE),
    (dict(eps=float("inf")), E_SHAPE),
    (dict(ws=None), E_WORKSPACE),
    (dict(wsb=8), E_WORKSPACE),
    (dict(ws=A + 4), E_ALIGN),
    (dict(K=48), E_SHAPE),
    (dict(n=1), E_PATTERN),
    (dict(bb=fp4(layout=1)), E_FORMAT),
])
def test_prep_rmsnorm_rejects(kwargs, status):
    assert prep_norm(**kwargs) == status


def test_prep_rmsnorm_workspace_and_device():
    L = sharq.lib()
    assert L.sharq_prep_rmsnorm_workspace_bytes(100, 64, 0) >= 100 * 4
    assert L.sharq_prep_rmsnorm_workspace_bytes(100, 64, 1) >= 100 * 4 + L.sharq_prep_workspace_bytes(100, 64, 1)
    import torch
    if not torch.cuda.is_available():
        assert prep_norm() == E_DEVICE


def test_binding_fails_loudly_without_the_library(monkeypatch):
    """No fallback: with the shared library absent every entry of the binding raises
    (there is no CPU path to fall back to)."""
    monkeypatch.setattr(sharq, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libsharq.so"))
    monkeypatch.setattr(sharq, "_lib", None)
    monkeypatch.setattr(sharq, "_raw", None)
    with pytest.raises(RuntimeError, match="missing"):
        sharq.lib()
    with pytest.raises(RuntimeError, match="missing"):
        sharq._raw_lib()
    with pytest.raises(RuntimeError, match="missing"):
        sharq.payload_sizes(16, 64, sharq.MXFP4, sharq.TILED)


def test_forward_noalloc_rejects_before_launch():
    """The allocation-free forward validates like sharq_forward before it touches the device."""
    L = sharq.lib()
    bb, rr, w = fp4(), fp4(), fp4()

    def call(**kw):
        a = dict(x=A, M=4, K=64, ldx=64, n=2, m=4, fmt=0, N=8, y=A, ldy=8, out=0)
        a.update(kw)
        return L.sharq_forward_noalloc(a["x"], a["M"], a["K"], a["ldx"], a["n"], a["m"], a["fmt"], ctypes.byref(bb),
                                       ctypes.byref(rr), ctypes.byref(w), a["N"], a["y"], a["ldy"], a["out"], None)
    assert call(ldy=4) == E_SHAPE
    assert call(out=9) == E_FORMAT
    assert call(n=1) == E_PATTERN
    assert call(y=None) == E_NULL
    assert call(fmt=7) == E_FORMAT
    assert call() == E_DEVICE  # valid arguments, no gfx950 in this process


def test_rounding_probe_rejects():
    L = sharq.lib()
    assert L.sharq_bf16_rounding_probe(None, None) == E_NULL
    assert L.sharq_bf16_rounding_probe(A + 4, None) == E_ALIGN
    assert L.sharq_e4m3_conversion_probe(None, None) == E_NULL
    assert L.sharq_e4m3_conversion_probe(A + 4, None) == E_ALIGN


def test_measurement_probes_reject():
    L = sharq.lib()
    assert L.sharq_matrix_rate_probe(2, 10, A, None) == E_FORMAT
    assert L.sharq_matrix_rate_probe(0, 10, None, None) == E_NULL
    assert L.sharq_matrix_rate_probe(1, 0, A, None) == E_SHAPE
    assert L.sharq_matrix_rate_probe(0, 10, A + 4, None) == E_ALIGN
    assert L.sharq_stream_probe(A, 17, A, 16, None) == E_SHAPE
    assert L.sharq_stream_probe(None, 16, A, 16, None) == E_NULL
    assert L.sharq_stream_probe(A + 8, 16, A, 16, None) == E_ALIGN
    assert L.sharq_stream_probe(A, 16, A, 16, None) == E_DEVICE

