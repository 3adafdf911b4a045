"""ctypes binding of libsharq (include/sharq.h).

Argument marshalling only: every step of the SharQ path runs in the HIP library.
PyTorch provides device memory and the current stream.  A missing library or a
non-zero status raises; there is no CPU fallback.
"""
import ctypes
import os

import torch

MXFP4 = 0
NVFP4 = 1
OUT_BF16 = 0
OUT_FP32 = 1
ROWMAJOR = 0
TILED = 1
BLOCK = {MXFP4: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsharq.so")

SYMBOLS = ["sharq_abi_version", "sharq_status_str", "sharq_payload_bytes", "sharq_convert_layout",
           "sharq_prep_workspace_bytes", "sharq_linear_workspace_bytes", "sharq_quantize", "sharq_prep",
           "sharq_prep_rmsnorm_workspace_bytes", "sharq_prep_rmsnorm", "sharq_linear", "sharq_linear_dense",
           "sharq_clock_probe", "sharq_prep_ablation", "sharq_dequantize", "sharq_prep_swiglu",
           "sharq_forward", "sharq_forward_noalloc", "sharq_matrix_rate_probe", "sharq_stream_probe",
           "sharq_bf16_rounding_probe", "sharq_e4m3_conversion_probe", "sharq_linear_split_workspace_bytes"]


class SharqFp4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SharqError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


ABI_VERSION = 12  # the SHARQ_ABI_VERSION of include/sharq.h this binding marshals for

_lib = None


def lib():
    """Load libsharq.so (built in-tree by build.py); raise if it is absent or was built
    for another ABI version than this binding's."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparsity_fp4_sharq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sharq_abi_version.restype = ctypes.c_int
        L.sharq_abi_version.argtypes = []
        found = L.sharq_abi_version()
        if found != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {found}, this binding expects {ABI_VERSION}: "
                               "rebuild the library")
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER(SharqFp4)
        L.sharq_abi_version.restype = ctypes.c_int
        L.sharq_abi_version.argtypes = []
        L.sharq_status_str.restype = ctypes.c_char_p
        L.sharq_status_str.argtypes = [ctypes.c_int]
        L.sharq_payload_bytes.restype = sz
        L.sharq_payload_bytes.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz),
                                          ctypes.POINTER(sz)]
        L.sharq_convert_layout.restype = ctypes.c_int
        L.sharq_convert_layout.argtypes = [P, P, i64, i64, ctypes.c_int, vp]
        L.sharq_prep_workspace_bytes.restype = sz
        L.sharq_prep_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
        L.sharq_linear_workspace_bytes.restype = sz
        L.sharq_linear_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
        L.sharq_linear_split_workspace_bytes.restype = sz
        L.sharq_linear_split_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
        L.sharq_quantize.restype = ctypes.c_int
        L.sharq_quantize.argtypes = [vp, i64, i64, i64, ctypes.c_int, P, vp, sz, vp]
        L.sharq_prep.restype = ctypes.c_int
        L.sharq_prep.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, vp,
                                 vp, sz, vp]
        L.sharq_prep_rmsnorm_workspace_bytes.restype = sz
        L.sharq_prep_rmsnorm_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
        L.sharq_prep_rmsnorm.restype = ctypes.c_int
        L.sharq_prep_rmsnorm.argtypes = [vp, i64, i64, i64, vp, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, P, P, vp, vp, sz, vp]
        L.sharq_linear.restype = ctypes.c_int
        L.sharq_linear.argtypes = [P, P, i64, P, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int, vp, sz,
                                   vp]
        L.sharq_linear_dense.restype = ctypes.c_int
        L.sharq_linear_dense.argtypes = [P, i64, P, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int, vp, sz, vp]
        L.sharq_prep_swiglu.restype = ctypes.c_int
        L.sharq_prep_swiglu.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, vp, vp,
                                        sz, vp]
        L.sharq_prep_ablation.restype = ctypes.c_int
        L.sharq_prep_ablation.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          P, P, vp, vp, sz, vp]
        L.sharq_dequantize.restype = ctypes.c_int
        L.sharq_dequantize.argtypes = [P, i64, i64, ctypes.c_int, vp, i64, vp]
        L.sharq_clock_probe.restype = ctypes.c_int
        L.sharq_clock_probe.argtypes = [i64, vp, vp]
        L.sharq_forward.restype = ctypes.c_int
        L.sharq_forward.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                    i64, vp, i64, ctypes.c_int, vp, sz, vp]
        L.sharq_matrix_rate_probe.restype = ctypes.c_int
        L.sharq_matrix_rate_probe.argtypes = [ctypes.c_int, i64, vp, vp]
        L.sharq_stream_probe.restype = ctypes.c_int
        L.sharq_stream_probe.argtypes = [vp, i64, vp, i64, vp]
        L.sharq_bf16_rounding_probe.restype = ctypes.c_int
        L.sharq_bf16_rounding_probe.argtypes = [vp, vp]
        L.sharq_e4m3_conversion_probe.restype = ctypes.c_int
        L.sharq_e4m3_conversion_probe.argtypes = [vp, vp]
        L.sharq_forward_noalloc.restype = ctypes.c_int
        L.sharq_forward_noalloc.argtypes = [vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                            i64, vp, i64, ctypes.c_int, vp]
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise SharqError(fn, status, lib().sharq_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def payload_sizes(rows, K, fmt, layout):
    """(codes bytes, scales bytes) of a payload, from the library."""
    c, sc = ctypes.c_size_t(0), ctypes.c_size_t(0)
    if lib().sharq_payload_bytes(rows, K, fmt, layout, ctypes.byref(c), ctypes.byref(sc)) == 0 and rows * K:
        raise ValueError(f"invalid payload: rows={rows} K={K} fmt={fmt} layout={layout}")
    return c.value, sc.value


def default_layout(fmt):
    return TILED if fmt == MXFP4 else ROWMAJOR


# ------------------------------------------------------------------ argument checks
# The C ABI receives raw pointers and cannot see buffer sizes, dtypes or devices, so the
# binding checks every buffer it passes before the foreign call (ValueError, nothing
# enqueued).

_REQUIRE_CUDA = True  # tensors must live on a GPU (the CPU tests of these checks lift it)


def _host_payload_sizes(rows, K, fmt, layout):
    """(codes bytes, scales bytes) of a payload, from the layouts of include/sharq.h."""
    if layout == TILED:
        rp, kp = -(-rows // 32) * 32, -(-K // 128) * 128
        return rp * kp // 2, rp * kp // 32
    return rows * K // 2, rows * K // BLOCK[fmt]


def _check_device(t, dev, what):
    if _REQUIRE_CUDA and not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{what} is on {t.device}, expected {dev}")


def _check_payload(p, fmt, rows, K, dev, what):
    if not isinstance(p, Payload):
        raise ValueError(f"{what} must be a Payload")
    if p.fmt != fmt:
        raise ValueError(f"{what} has format {p.fmt}, expected {fmt}")
    if p.rows != rows or p.K != K:
        raise ValueError(f"{what} is [{p.rows}, {p.K}], expected [{rows}, {K}]")
    if p.layout not in (ROWMAJOR, TILED) or (p.layout == TILED and fmt != MXFP4):
        raise ValueError(f"{what} has an invalid layout {p.layout} for format {fmt}")
    if fmt not in BLOCK or K <= 0 or K % BLOCK[fmt] or rows < 0:
        raise ValueError(f"{what}: invalid shape [{rows}, {K}] for format {fmt}")
    cb, sb = _host_payload_sizes(rows, K, fmt, p.layout)
    for t, need, name in ((p.codes, cb, "codes"), (p.scales, sb, "scales")):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{what}.{name} must be a contiguous uint8 tensor")
        if t.numel() < need:
            raise ValueError(f"{what}.{name} holds {t.numel()} bytes, needs {need}")
        _check_device(t, dev, f"{what}.{name}")
    ts = p.tensor_scale
    if ts is None or ts.dtype != torch.float32 or ts.numel() < 1:
        raise ValueError(f"{what}.tensor_scale must be a float32 tensor of at least one element")
    _check_device(ts, dev, f"{what}.tensor_scale")


def _check_output(y, M, N, out_dtype, dev):
    want = {OUT_FP32: torch.float32, OUT_BF16: torch.bfloat16}.get(out_dtype)
    if want is None:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    if y.dtype != want:
        raise ValueError(f"y has dtype {y.dtype}, out_dtype {out_dtype} writes {want}")
    if y.dim() != 2 or tuple(y.shape) != (M, N):
        raise ValueError(f"y has shape {tuple(y.shape)}, expected ({M}, {N})")
    if M > 0 and y.stride(1) != 1:
        raise ValueError("y must have a unit column stride")
    if M > 1 and y.stride(0) < N:
        raise ValueError("y rows overlap (row stride < N)")
    _check_device(y, dev, "y")


def _check_workspace(ws, need, dev):
    if need == 0 and ws is None:
        return
    if ws is None:
        raise ValueError(f"a workspace of {need} bytes is required")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("the workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"the workspace holds {ws.numel()} bytes, needs {need}")
    _check_device(ws, dev, "workspace")


class Payload:
    """Device FP4 tensor [rows, K]: flat uint8 codes and scales in `layout`, plus a
    float32 tensor scale (NVFP4)."""

    def __init__(self, codes, scales, tensor_scale, fmt, layout=ROWMAJOR, rows=None, K=None):
        self.codes, self.scales, self.tensor_scale, self.fmt, self.layout = codes, scales, tensor_scale, fmt, layout
        self.rows = codes.shape[0] if rows is None else rows
        self.K = codes.shape[1] * 2 if K is None else K

    @classmethod
    def empty(cls, rows, K, fmt, device, layout=None):
        layout = default_layout(fmt) if layout is None else layout
        cb, sb = payload_sizes(rows, K, fmt, layout)
        codes = torch.empty(cb, dtype=torch.uint8, device=device)
        scales = torch.empty(sb, dtype=torch.uint8, device=device)
        ts = torch.empty(4, dtype=torch.float32, device=device)  # 16 bytes, first element used
        return cls(codes, scales, ts, fmt, layout, rows, K)

    def struct(self):
        return SharqFp4(self.codes.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr(),
                        self.layout, 0)

    def convert(self, layout, stream=None):
        """This payload in another layout (a new payload; on-device re-layout)."""
        _check_payload(self, self.fmt, self.rows, self.K, self.codes.device, "payload")
        out = Payload.empty(self.rows, self.K, self.fmt, self.codes.device, layout)
        src, dst = self.struct(), out.struct()
        _check("sharq_convert_layout", lib().sharq_convert_layout(ctypes.byref(src), ctypes.byref(dst), self.rows,
                                                                  self.K, self.fmt, _stream(stream)))
        if self.fmt == NVFP4:
            out.tensor_scale.copy_(self.tensor_scale)
        return out

    def to_host(self):
        """(codes [rows, K/2], scales [rows, K/B], tensor scale) as numpy, row-major."""
        p = self if self.layout == ROWMAJOR else self.convert(ROWMAJOR)
        ts = float(p.tensor_scale[0].item()) if p.fmt == NVFP4 else 1.0
        codes = p.codes.cpu().numpy().reshape(p.rows, p.K // 2)
        scales = p.scales.cpu().numpy().reshape(p.rows, p.K // BLOCK[p.fmt])
        return codes, scales, ts

    def raw_host(self):
        """The raw device bytes (codes, scales) as numpy, in this payload's layout."""
        return self.codes.cpu().numpy(), self.scales.cpu().numpy()


def workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def _as_bf16_2d(x):
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("expected a 2-D bfloat16 tensor")
    _check_device(x, None, "x")
    if x.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return x


def _prep_outputs(out, M, K, fmt, dev, layout):
    bb, rr = out if out is not None else (Payload.empty(M, K, fmt, dev, layout),
                                          Payload.empty(M, K, fmt, dev, layout))
    _check_payload(bb, fmt, M, K, dev, "backbone")
    _check_payload(rr, fmt, M, K, dev, "residual")
    if bb.layout != rr.layout:
        raise ValueError("backbone and residual must share a layout")
    return bb, rr


def quantize(x, fmt=MXFP4, layout=None, stream=None, out=None, ws=None):
    """Plain FP4 quantization of a bf16 matrix (a weight payload, or the activation of
    a plain FP4 layer)."""
    x = _as_bf16_2d(x)
    rows, K = x.shape
    if out is None:
        out = Payload.empty(rows, K, fmt, x.device, layout)
    _check_payload(out, fmt, rows, K, x.device, "out")
    need = lib().sharq_prep_workspace_bytes(rows, K, fmt)
    if ws is None:
        ws = workspace(need, x.device)
    _check_workspace(ws, need, x.device)
    st = out.struct()
    _check("sharq_quantize", lib().sharq_quantize(_ptr(x), rows, K, x.stride(0), fmt, ctypes.byref(st),
                                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out


def prep(x, n=2, m=4, fmt=MXFP4, want_mask=False, out=None, ws=None, layout=None, stream=None):
    """SharQ activation preparation: returns (backbone, residual, mask_bits or None)."""
    x = _as_bf16_2d(x)
    M, K = x.shape
    bb, rr = _prep_outputs(out, M, K, fmt, x.device, layout)
    mask = torch.empty((M, K // 8), dtype=torch.uint8, device=x.device) if want_mask else None
    need = lib().sharq_prep_workspace_bytes(M, K, fmt)
    if ws is None:
        ws = workspace(need, x.device)
    _check_workspace(ws, need, x.device)
    sb, sr = bb.struct(), rr.struct()
    _check("sharq_prep", lib().sharq_prep(_ptr(x), M, K, x.stride(0), n, m, fmt, ctypes.byref(sb),
                                          ctypes.byref(sr), _ptr(mask), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(stream)))
    return bb, rr, mask


def prep_rmsnorm(x, gamma, eps=1e-6, n=2, m=4, fmt=MXFP4, want_mask=False, out=None, ws=None, layout=None,
                 stream=None):
    """SharQ preparation of RMSNorm(x) * gamma (bf16 gains [K]): returns (backbone,
    residual, mask_bits or None)."""
    x = _as_bf16_2d(x)
    M, K = x.shape
    if gamma.dtype != torch.bfloat16 or gamma.dim() != 1 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bfloat16 vector of K entries")
    _check_device(gamma, x.device, "gamma")
    bb, rr = _prep_outputs(out, M, K, fmt, x.device, layout)
    mask = torch.empty((M, K // 8), dtype=torch.uint8, device=x.device) if want_mask else None
    need = lib().sharq_prep_rmsnorm_workspace_bytes(M, K, fmt)
    if ws is None:
        ws = workspace(need, x.device)
    _check_workspace(ws, need, x.device)
    sb, sr = bb.struct(), rr.struct()
    _check("sharq_prep_rmsnorm", lib().sharq_prep_rmsnorm(_ptr(x), M, K, x.stride(0), _ptr(gamma), float(eps), n, m,
                                                          fmt, ctypes.byref(sb), ctypes.byref(sr), _ptr(mask),
                                                          _ptr(ws), 0 if ws is None else ws.numel(),
                                                          _stream(stream)))
    return bb, rr, mask


def linear(backbone, residual, weight, out_dtype=OUT_BF16, y=None, ws=None, stream=None):
    """Y = Bhat W^T + Rhat W^T on the device; returns Y [M, N] (bf16 or fp32)."""
    fmt = weight.fmt
    M, K, N = backbone.rows, backbone.K, weight.rows
    dev = weight.codes.device
    _check_payload(weight, fmt, N, K, dev, "weight")
    _check_payload(backbone, fmt, M, K, dev, "backbone")
    _check_payload(residual, fmt, M, K, dev, "residual")
    if not backbone.layout == residual.layout == weight.layout:
        raise ValueError("backbone, residual and weight must share a layout")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16, device=dev)
    _check_output(y, M, N, out_dtype, dev)
    need = lib().sharq_linear_workspace_bytes(M, N, K, fmt)
    if ws is None:  # with room for the K split where the shape has one
        ws = workspace(max(need, lib().sharq_linear_split_workspace_bytes(M, N, K, fmt)), dev)
    _check_workspace(ws, need, dev)
    sb, sr, sw = backbone.struct(), residual.struct(), weight.struct()
    _check("sharq_linear", lib().sharq_linear(ctypes.byref(sb), ctypes.byref(sr), M, ctypes.byref(sw), N, K,
                                              fmt, _ptr(y), y.stride(0), out_dtype, _ptr(ws),
                                              0 if ws is None else ws.numel(), _stream(stream)))
    return y


def linear_dense(a, weight, out_dtype=OUT_BF16, y=None, ws=None, stream=None):
    """Plain FP4 linear Y = Ahat W^T (no SharQ) on the device; returns Y [M, N]."""
    fmt = weight.fmt
    M, K, N = a.rows, a.K, weight.rows
    dev = weight.codes.device
    _check_payload(weight, fmt, N, K, dev, "weight")
    _check_payload(a, fmt, M, K, dev, "a")
    if a.layout != weight.layout:
        raise ValueError("a and weight must share a layout")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16, device=dev)
    _check_output(y, M, N, out_dtype, dev)
    need = lib().sharq_linear_workspace_bytes(M, N, K, fmt)
    if ws is None:  # with room for the K split where the shape has one
        ws = workspace(max(need, lib().sharq_linear_split_workspace_bytes(M, N, K, fmt)), dev)
    _check_workspace(ws, need, dev)
    sa, sw = a.struct(), weight.struct()
    _check("sharq_linear_dense", lib().sharq_linear_dense(ctypes.byref(sa), M, ctypes.byref(sw), N, K, fmt, _ptr(y),
                                                          y.stride(0), out_dtype, _ptr(ws),
                                                          0 if ws is None else ws.numel(), _stream(stream)))
    return y


def prep_swiglu(gate_up, I, n=2, m=4, fmt=MXFP4, want_mask=False, out=None, ws=None, layout=None, stream=None):
    """SharQ preparation of h = SwiGLU(gate, up) for gate_up bf16 [M, ld >= 2I] (gate in
    columns [0, I), up in [I, 2I)): returns (backbone, residual, mask_bits or None)."""
    if gate_up.dtype != torch.bfloat16 or gate_up.dim() != 2 or gate_up.stride(1) != 1:
        raise ValueError("gate_up must be a 2-D bf16 tensor with unit column stride")
    _check_device(gate_up, None, "gate_up")
    M = gate_up.shape[0]
    if gate_up.shape[1] < 2 * I:
        raise ValueError("gate_up needs at least 2*I columns")
    bb, rr = _prep_outputs(out, M, I, fmt, gate_up.device, layout)
    mask = torch.empty((M, I // 8), dtype=torch.uint8, device=gate_up.device) if want_mask else None
    need = lib().sharq_prep_workspace_bytes(M, I, fmt)
    if ws is None:
        ws = workspace(need, gate_up.device)
    _check_workspace(ws, need, gate_up.device)
    sb, sr = bb.struct(), rr.struct()
    _check("sharq_prep_swiglu", lib().sharq_prep_swiglu(_ptr(gate_up), M, I, gate_up.stride(0), n, m, fmt,
                                                        ctypes.byref(sb), ctypes.byref(sr), _ptr(mask), _ptr(ws),
                                                        0 if ws is None else ws.numel(), _stream(stream)))
    return bb, rr, mask


ABLATE_RESIDUAL_UNQUANTIZED = 1
ABLATE_STATIC_MASK = 2
ABLATE_NO_RESIDUAL = 3


def prep_ablation(x, variant, n=2, m=4, fmt=MXFP4, want_mask=False, out=None, ws=None, layout=None, stream=None):
    """sharq_prep with one of the ablations (ABLATE_*): returns (backbone, residual, mask_bits or None)."""
    x = _as_bf16_2d(x)
    M, K = x.shape
    bb, rr = _prep_outputs(out, M, K, fmt, x.device, layout)
    mask = torch.empty((M, K // 8), dtype=torch.uint8, device=x.device) if want_mask else None
    need = lib().sharq_prep_workspace_bytes(M, K, fmt)
    if ws is None:
        ws = workspace(need, x.device)
    _check_workspace(ws, need, x.device)
    sb, sr = bb.struct(), rr.struct()
    _check("sharq_prep_ablation", lib().sharq_prep_ablation(_ptr(x), M, K, x.stride(0), n, m, fmt, variant,
                                                            ctypes.byref(sb), ctypes.byref(sr), _ptr(mask), _ptr(ws),
                                                            0 if ws is None else ws.numel(), _stream(stream)))
    return bb, rr, mask


def dequantize(p, out=None, stream=None):
    """fp32 values [rows, K] of a payload, on the device."""
    dev = p.codes.device
    _check_payload(p, p.fmt, p.rows, p.K, dev, "payload")
    if out is None:
        out = torch.empty((p.rows, p.K), dtype=torch.float32, device=dev)
    _check_output(out, p.rows, p.K, OUT_FP32, dev)
    st = p.struct()
    _check("sharq_dequantize", lib().sharq_dequantize(ctypes.byref(st), p.rows, p.K, p.fmt, _ptr(out), out.stride(0),
                                                      _stream(stream)))
    return out


def clock_probe(iters=20000, device=None, stream=None):
    """Shader clock (Hz) under FP4 matrix load, from the device's cycle and 100 MHz counters."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    _check("sharq_clock_probe", lib().sharq_clock_probe(iters, _ptr(out), _stream(stream)))
    cycles, ticks = (int(v) for v in out[:2].cpu())
    return cycles / (ticks / 1e8) if ticks > 0 else float("nan")


def _forward_args(x, weight, out_dtype, bufs, y, ws, with_workspace=True):
    """Buffers of one forward call, allocated where absent and checked (no workspace when
    with_workspace is false)."""
    x = _as_bf16_2d(x)
    fmt = weight.fmt
    M, K = x.shape
    N = weight.rows
    dev = x.device
    _check_payload(weight, fmt, N, K, dev, "weight")
    bb, rr = _prep_outputs(bufs, M, K, fmt, dev, weight.layout)
    if bb.layout != weight.layout:
        raise ValueError("the activation payloads and the weight must share a layout")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16, device=dev)
    _check_output(y, M, N, out_dtype, dev)
    if with_workspace:
        need = max(lib().sharq_prep_workspace_bytes(M, K, fmt), lib().sharq_linear_workspace_bytes(M, N, K, fmt))
        if ws is None:  # with room for the K split where the shape has one
            ws = workspace(max(need, lib().sharq_linear_split_workspace_bytes(M, N, K, fmt)), dev)
        _check_workspace(ws, need, dev)
    return x, bb, rr, y, ws, M, K, N, fmt


def matrix_rate_probe(form, iters=20000, device=None, stream=None):
    """Issue rate of a matrix-instruction form (0: dense scaled FP4 32x32x64, 1: 2:4-sparse
    fp8 32x32x64): returns (cycles per instruction per SIMD, shader clock in Hz)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    _check("sharq_matrix_rate_probe", lib().sharq_matrix_rate_probe(form, iters, _ptr(out), _stream(stream)))
    cycles, ticks = (int(v) for v in out[:2].cpu())
    return cycles / (iters * 8), (cycles / (ticks / 1e8) if ticks > 0 else float("nan"))


def stream_probe(src, read_bytes, dst, write_bytes, stream=None):
    """A plain read of read_bytes of src and write of write_bytes of dst (uint8 CUDA tensors)."""
    for t, n, what in ((src, read_bytes, "src"), (dst, write_bytes, "dst")):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{what} must be a contiguous uint8 tensor of at least {n} bytes")
        _check_device(t, src.device, what)
    _check("sharq_stream_probe", lib().sharq_stream_probe(_ptr(src), read_bytes, _ptr(dst), write_bytes,
                                                          _stream(stream)))


def bf16_rounding_probe(device=None, stream=None):
    """Every fp32 pattern through the device's packed bf16 conversion: returns (number of
    finite patterns that differ from round-to-nearest-even on the bits, smallest one)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    _check("sharq_bf16_rounding_probe", lib().sharq_bf16_rounding_probe(_ptr(out), _stream(stream)))
    bad, first = (int(v) & 0xFFFFFFFFFFFFFFFF for v in out.cpu())
    return bad, first


def e4m3_conversion_probe(device=None, stream=None):
    """The device's E4M3 conversions against the format's definition: returns (number of
    mismatches over every non-negative fp32 operand and every code 0..0x7E, smallest
    mismatching pattern, or 2^32 + code for a decode)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    _check("sharq_e4m3_conversion_probe", lib().sharq_e4m3_conversion_probe(_ptr(out), _stream(stream)))
    bad, first = (int(v) & 0xFFFFFFFFFFFFFFFF for v in out.cpu())
    return bad, first


_raw = None


def _raw_lib():
    """The library through a second handle with no argtypes: calls pass ctypes instances
    through unconverted (for pre-marshalled calls)."""
    global _raw
    if _raw is None:
        lib()  # checks presence and the ABI version
        _raw = ctypes.CDLL(LIB_PATH)
    return _raw


def bind_forward(x, weight, n=2, m=4, out_dtype=OUT_BF16, bufs=None, y=None, ws=None, stream=None):
    """`forward` with its arguments marshalled once: returns a zero-argument callable that
    issues the same sharq_forward on the same buffers and stream (one foreign call per
    invocation, for launch-bound shapes such as decode).  The callable keeps the buffers
    alive; its `outputs` attribute is (y, (backbone, residual)).  A non-zero status raises
    SharqError at the call."""
    x, bb, rr, y, ws, M, K, N, fmt = _forward_args(x, weight, out_dtype, bufs, y, ws)
    sb, sr, sw = bb.struct(), rr.struct(), weight.struct()
    i64, ci = ctypes.c_int64, ctypes.c_int
    args = (ctypes.c_void_p(x.data_ptr()), i64(M), i64(K), i64(x.stride(0)), ci(n), ci(m), ci(fmt),
            ctypes.byref(sb), ctypes.byref(sr), ctypes.byref(sw), i64(N), ctypes.c_void_p(y.data_ptr()),
            i64(y.stride(0)), ci(out_dtype), _ptr(ws), ctypes.c_size_t(0 if ws is None else ws.numel()),
            _stream(stream))
    fn = _raw_lib().sharq_forward
    keep = (x, weight, bb, rr, y, ws, sb, sr, sw)

    def call():
        status = fn(*args)
        if status != 0:
            _check("sharq_forward", status)

    call.outputs = (y, (bb, rr))
    call._keep = keep
    return call


def forward(x, weight, n=2, m=4, out_dtype=OUT_BF16, bufs=None, y=None, ws=None, stream=None):
    """One SharQ linear layer: prep then both GEMMs, on one stream."""
    x, bb, rr, y, ws, M, K, N, fmt = _forward_args(x, weight, out_dtype, bufs, y, ws)
    sb, sr, sw = bb.struct(), rr.struct(), weight.struct()
    _check("sharq_forward", lib().sharq_forward(_ptr(x), M, K, x.stride(0), n, m, fmt, ctypes.byref(sb),
                                                ctypes.byref(sr), ctypes.byref(sw), N, _ptr(y), y.stride(0),
                                                out_dtype, _ptr(ws), 0 if ws is None else ws.numel(),
                                                _stream(stream)))
    return y, (bb, rr)


def forward_noalloc(x, weight, n=2, m=4, out_dtype=OUT_BF16, bufs=None, y=None, stream=None):
    """`forward` through sharq_forward_noalloc: the library's fixed per-device scratch in
    place of a workspace (the caller still passes, or here lets the binding allocate,
    the inputs and outputs).  Calls on one GPU share that scratch: do not overlap them."""
    x, bb, rr, y, _, M, K, N, fmt = _forward_args(x, weight, out_dtype, bufs, y, None, with_workspace=False)
    sb, sr, sw = bb.struct(), rr.struct(), weight.struct()
    _check("sharq_forward_noalloc", lib().sharq_forward_noalloc(_ptr(x), M, K, x.stride(0), n, m, fmt,
                                                                ctypes.byref(sb), ctypes.byref(sr), ctypes.byref(sw),
                                                                N, _ptr(y), y.stride(0), out_dtype, _stream(stream)))
    return y, (bb, rr)
