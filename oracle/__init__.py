"""CPU oracle for the SharQ sparse-dense FP4 linear layer -- TEST INFRASTRUCTURE ONLY.

Thin ctypes marshalling over ``liboracle.so`` (built from ``sharq_oracle.c``).
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP library and never imports it.

All arrays are numpy; bf16 tensors travel as ``uint16`` bit patterns.
Parity status: every function here is pinned by the CPU tests (brute force,
closed forms, exact rational arithmetic, invariants, hand-worked examples).  The
NVFP4 rule is a reading of the pages (they name the format, not its arithmetic);
two hand-worked NVFP4 examples fix its fp32 rounding sequence step by step, and a
test plants each plausible deviation from it in a copy of the oracle and sees an
example fail (likewise for the mask, the MX scale and rounding, the residual, the
packing, the GEMM, the RMS normalization and the SwiGLU).
"""
import ctypes
import os

import numpy as np

MXFP4 = 0
NVFP4 = 1
BLOCK = {MXFP4: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it with gcc when it is absent or older than its source."""
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "sharq_oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_mx_exponent.restype = ctypes.c_int
        L.oracle_mx_exponent.argtypes = [ctypes.c_double]
        L.oracle_nv_tensor_scale.restype = ctypes.c_float
        L.oracle_nv_tensor_scale.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_array.restype = None
        L.oracle_e2m1_encode_array.argtypes = [_f32p, _i64, _u8p]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_encode_array.argtypes = [_f32p, _i64, _u8p]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int, _u8p, _u8p, _vp]
        L.oracle_prep.restype = ctypes.c_int
        L.oracle_prep.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  _u8p, _u8p, _vp, _u8p, _u8p, _vp, _vp, _vp, _vp]
        L.oracle_prep_variant.restype = ctypes.c_int
        L.oracle_prep_variant.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _u8p, _u8p, _vp, _u8p, _u8p, _vp, _vp, _vp, _vp]
        L.oracle_silu.restype = ctypes.c_float
        L.oracle_silu.argtypes = [ctypes.c_float]
        L.oracle_swiglu.restype = ctypes.c_int
        L.oracle_swiglu.argtypes = [_u16p, _i64, _i64, _i64, _u16p]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_dequant.argtypes = [_u8p, _u8p, ctypes.c_float, _i64, _i64, ctypes.c_int, _f64p]
        L.oracle_linear.restype = ctypes.c_int
        L.oracle_linear.argtypes = [_u8p, _u8p, ctypes.c_float, _u8p, _u8p, ctypes.c_float, _i64,
                                    _u8p, _u8p, ctypes.c_float, _i64, _i64, ctypes.c_int, _vp, _i64,
                                    _f64p]
        L.oracle_row_sumsq.restype = ctypes.c_int
        L.oracle_row_sumsq.argtypes = [_u16p, _i64, _i64, _i64, _f64p]
        L.oracle_rmsnorm.restype = ctypes.c_int
        L.oracle_rmsnorm.argtypes = [_u16p, _i64, _i64, _i64, _u16p, ctypes.c_float, _u16p, _vp]
        L.oracle_omp_threads.restype = ctypes.c_int
        L.oracle_omp_threads.argtypes = []
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Payload:
    """An FP4 tensor: codes [rows, K/2] uint8, scales [rows, K/B] uint8, tensor scale."""

    def __init__(self, codes, scales, tscale=1.0):
        self.codes = codes
        self.scales = scales
        self.tscale = float(tscale)

    def __repr__(self):
        return f"Payload(codes={self.codes.shape}, scales={self.scales.shape}, tscale={self.tscale})"


def _alloc(rows, K, fmt):
    return (np.zeros((rows, K // 2), np.uint8), np.zeros((rows, K // BLOCK[fmt]), np.uint8))


def quantize(x_bits, fmt=MXFP4):
    """Plain FP4 quantization of a bf16 matrix (uint16 bits [rows, K])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, K = x_bits.shape
    codes, scales = _alloc(rows, K, fmt)
    ts = np.ones(1, np.float32)
    rc = lib().oracle_quantize(x_bits, rows, K, K, fmt, codes, scales, _ptr(ts))
    if rc:
        raise ValueError(f"oracle_quantize rejected shape {x_bits.shape} fmt {fmt}")
    return Payload(codes, scales, ts[0])


def silu(g):
    """silu(g) in fp32 by reading R14 (scalar)."""
    return float(lib().oracle_silu(float(g)))


def swiglu(gate_up_bits, I):
    """bf16 h [M, I] = bf16(fp32(silu(gate) * up)) of gate_up [M, ld >= 2I] (gate in
    columns [0, I), up in [I, 2I)), reading R14."""
    gu = np.ascontiguousarray(gate_up_bits, dtype=np.uint16)
    M, ld = gu.shape
    h = np.zeros((M, I), np.uint16)
    if lib().oracle_swiglu(gu, M, I, ld, h):
        raise ValueError("oracle_swiglu rejected its arguments")
    return h


def row_sumsq(x_bits):
    """fp64 sums of squares of the rows of a bf16 matrix, in reading R9's order."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    out = np.zeros(max(M, 1), np.float64)
    if lib().oracle_row_sumsq(x_bits, M, K, K, out):
        raise ValueError("oracle_row_sumsq rejected its arguments")
    return out[:M]


def rmsnorm(x_bits, gamma_bits, eps):
    """RMS normalization with a bf16 gain (reading R9): returns (y bf16 bits [M, K],
    the per-row factors r as float32 [M])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    gamma_bits = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if gamma_bits.shape != (K,):
        raise ValueError("gamma must have K entries")
    y = np.zeros((M, K), np.uint16)
    r = np.zeros(max(M, 1), np.float32)
    rc = lib().oracle_rmsnorm(x_bits, M, K, K, gamma_bits, float(eps), y, _ptr(r))
    if rc:
        raise ValueError("oracle_rmsnorm rejected its arguments")
    return y, r[:M]


ABLATE_RESIDUAL_UNQUANTIZED = 1
ABLATE_STATIC_MASK = 2
ABLATE_NO_RESIDUAL = 3


def prep(x_bits, n, m, fmt=MXFP4, want_values=False, variant=0):
    """SharQ activation preparation.  Returns (backbone, residual, mask_bits[, bhat, resid]).
    variant: 0 = the method; 1-3 = the ablations of reading R13 (residual against the
    unquantized sparse values, static mask, no residual)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    bc, bs = _alloc(M, K, fmt)
    rc_, rs = _alloc(M, K, fmt)
    bt = np.ones(1, np.float32)
    rt = np.ones(1, np.float32)
    mask = np.zeros((M, K // 8), np.uint8)
    bh = np.zeros((M, K), np.float32) if want_values else None
    rr = np.zeros((M, K), np.float32) if want_values else None
    rc = lib().oracle_prep_variant(x_bits, M, K, K, n, m, fmt, variant, bc, bs, _ptr(bt), rc_, rs, _ptr(rt),
                           _ptr(mask), _ptr(bh), _ptr(rr))
    if rc:
        raise ValueError(f"oracle_prep rejected shape {x_bits.shape} pattern {n}:{m} fmt {fmt}")
    out = (Payload(bc, bs, bt[0]), Payload(rc_, rs, rt[0]), mask)
    if want_values:
        out = out + (bh, rr)
    return out


def dequant(p, fmt=MXFP4):
    """Exact fp64 values of an FP4 payload."""
    rows = p.codes.shape[0]
    K = p.codes.shape[1] * 2
    out = np.zeros((rows, K), np.float64)
    rc = lib().oracle_dequant(np.ascontiguousarray(p.codes), np.ascontiguousarray(p.scales),
                              p.tscale, rows, K, fmt, out)
    if rc:
        raise ValueError("oracle_dequant rejected its arguments")
    return out


def linear(backbone, residual, weight, fmt=MXFP4, rows=None):
    """Y = Bhat W^T + Rhat W^T in fp64, for all rows or the selected row indices."""
    M = backbone.codes.shape[0]
    K = backbone.codes.shape[1] * 2
    N = weight.codes.shape[0]
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_sel = M if sel is None else len(sel)
    y = np.zeros((n_sel, N), np.float64)
    rc = lib().oracle_linear(backbone.codes, backbone.scales, backbone.tscale,
                             residual.codes, residual.scales, residual.tscale, M,
                             weight.codes, weight.scales, weight.tscale, N, K, fmt,
                             _ptr(sel), n_sel, y)
    if rc:
        raise ValueError("oracle_linear rejected its arguments")
    return y


def linear_dense(a, weight, fmt=MXFP4, rows=None):
    """Plain FP4 linear Y = Ahat W^T in fp64 (no SharQ decomposition): the GEMM pair
    above with an all-zero backbone payload, whose every product is an exact zero."""
    zero = Payload(np.zeros_like(a.codes), np.zeros_like(a.scales), 1.0)
    return linear(zero, a, weight, fmt, rows)


def e2m1_encode(t):
    t = np.ascontiguousarray(t, dtype=np.float32).ravel()
    out = np.zeros(t.size, np.uint8)
    lib().oracle_e2m1_encode_array(t, t.size, out)
    return out


def e4m3_encode(q):
    q = np.ascontiguousarray(q, dtype=np.float32).ravel()
    out = np.zeros(q.size, np.uint8)
    lib().oracle_e4m3_encode_array(q, q.size, out)
    return out


def mx_exponent(amax):
    return lib().oracle_mx_exponent(float(amax))


def threads():
    return lib().oracle_omp_threads()


def set_threads(n):
    """Thread count of the oracle's row loops (for timing only)."""
    lib().oracle_set_threads(int(n))
