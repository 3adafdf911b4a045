"""The worked examples pin the oracle's readings: each test below plants one
plausible deviation in a temporary copy of the oracle's C source (on the CPU),
builds it, and checks that a stored worked example then fails.  The NVFP4
examples pin reading R5's fp32 steps; the MXFP4 examples pin the mask (R1), the
E8M0 block exponent (R2), E2M1 rounding (R3), the residual taken against the
dequantized backbone (R4) and the nibble packing (R6).

R5 (NVFP4 with per-path tensor scales; SharQ, arXiv 2606.26587, abstract: the
method runs on NVFP4 and names path-specific scale views): S = fp32(amax/2688),
q = fp32(amax_blk / fp32(6 S)), s = E4M3(q), d = fp32(s S),
code = E2M1(fp32(x / d)), Bhat = fp32(v d), R = fp32(x - Bhat).
The stored values come from tests/golden/hand_examples.json; none of them was
produced by the oracle.
"""
import ctypes
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from activation_sparsity_fp4_sharq_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "sharq_oracle.c")
GOLDEN = os.path.join(HERE, "golden", "hand_examples.json")

# (name, text of R5's step in the oracle, the same step with the deviation)
MUTATIONS = [
    ("6S unrounded", "  float q = amax / six_s;",
     "  float q = (float)((double)amax / (6.0 * (double)S));"),
    ("division reordered as (amax/6)/S", "  float q = amax / six_s;",
     "  float q = (amax / 6.0f) / S;"),
    ("q unrounded before E4M3", "  uint8_t sb = oracle_e4m3_encode(q);",
     "  uint8_t sb = oracle_e4m3_encode_exact((double)amax / (double)six_s);"),
    ("d unrounded", "      float t = v[i] / d;",
     "      float t = (float)((double)v[i] / (oracle_e4m3_value(sb) * (double)S));"),
    ("x/d unrounded (fp64 quotient)", "      codes[i] = oracle_e2m1_encode((double)t);",
     "      codes[i] = oracle_e2m1_encode((double)v[i] / (double)d); (void)t;"),
    ("R by fused multiply-add", "        float r = xv - bh;",
     "        float r = fmt == ORACLE_MXFP4 ? xv - bh : fmaf(-(float)oracle_e2m1_value(c[j]),"
     " (float)oracle_e4m3_value(sb) * Sb, xv);"),
]

# (name, text of the step in the oracle, the same step with the deviation): readings
# R1-R4 and R6 of the MXFP4 path (SharQ, arXiv 2606.26587, abstract and Core claim:
# an input-adaptive N:M mask keeps the outlier-dominated values, the residual is taken
# against the quantized backbone; the block format is the OCP MX rule the page cites)
MX_MUTATIONS = [
    ("mask ties to the higher index", "      if (kl > kj || (kl == kj && l < j)) ++rank;",
     "      if (kl > kj || (kl == kj && l > j)) ++rank;"),
    ("mask on signed values instead of magnitudes",
     "    uint16_t kj = xg[j] & 0x7FFF;\n    int rank = 0;\n    for (int l = 0; l < m; ++l) {\n"
     "      uint16_t kl = xg[l] & 0x7FFF;",
     "    uint16_t kj = (xg[j] & 0x8000) ? (uint16_t)(0x7FFF - (xg[j] & 0x7FFF)) : (uint16_t)(xg[j] | 0x8000);\n"
     "    int rank = 0;\n    for (int l = 0; l < m; ++l) {\n"
     "      uint16_t kl = (xg[l] & 0x8000) ? (uint16_t)(0x7FFF - (xg[l] & 0x7FFF)) : (uint16_t)(xg[l] | 0x8000);"),
    ("mask keeps the smallest magnitudes", "    keep[j] = rank < n;", "    keep[j] = rank >= m - n;"),
    ("block exponent floor(log2 amax) - 1", "  int e = (e2 - 1) - 2;", "  int e = (e2 - 1) - 1;"),
    ("block exponent ceil(log2 amax) - 2", "  int e = (e2 - 1) - 2;",
     "  int e = (frexp(amax, &e2) == 0.5 ? e2 - 1 : e2) - 2;"),
    ("E2M1 ties away from zero", "    if (a > mid || (a == mid && (upper & 1) == 0)) mag = (uint8_t)upper;",
     "    if (a >= mid) mag = (uint8_t)upper;"),
    ("E2M1 ties toward zero", "    if (a > mid || (a == mid && (upper & 1) == 0)) mag = (uint8_t)upper;",
     "    if (a > mid) mag = (uint8_t)upper;"),
    ("E2M1 drops the sign of a value rounding to zero", "  return (uint8_t)((signbit(t) ? 8 : 0) | mag);",
     "  return (uint8_t)((signbit(t) && mag ? 8 : 0) | mag);"),
    ("residual against the unquantized sparse values", "        float r = xv - bh;                                            /* R4 */",
     "        float r = xv - (keep[i * K + k0 + j] ? xv : 0.0f); (void)bh;"),
    ("dequantization off by one binade", "  return (float)ldexp(oracle_e2m1_value(code), (int)scale_byte - 127);",
     "  return (float)ldexp(oracle_e2m1_value(code), (int)scale_byte - 128);"),
    ("nibbles packed high first", "  if (k & 1) *b = (uint8_t)((*b & 0x0F) | (code << 4));\n  else *b = (uint8_t)((*b & 0xF0) | (code & 0x0F));",
     "  if (!(k & 1)) *b = (uint8_t)((*b & 0x0F) | (code << 4));\n  else *b = (uint8_t)((*b & 0xF0) | (code & 0x0F));"),
]

# an E4M3 encoder of an unrounded quotient, for the "q unrounded" deviation
EXACT_ENCODER = r"""
static uint8_t oracle_e4m3_encode_exact(double q) {
  if (!(q > 0.0)) return 0;
  if (q >= 448.0) return 0x7E;
  int e2;
  (void)frexp(q, &e2);
  int e = e2 - 1;
  double step = (e < -6) ? ldexp(1.0, -9) : ldexp(1.0, e - 3);
  double v = nearbyint(q / step) * step;
  if (v >= 448.0) return 0x7E;
  if (v == 0.0) return 0;
  (void)frexp(v, &e2);
  e = e2 - 1;
  if (e < -6) return (uint8_t)(v / ldexp(1.0, -9));
  return (uint8_t)(((e + 7) << 3) | (int)((v / ldexp(1.0, e) - 1.0) * 8.0));
}
"""


def _examples(fmt):
    with open(GOLDEN) as f:
        return [e for e in json.load(f)["examples"] if e["fmt"] == fmt]


def _nv_examples():
    return _examples("nvfp4")


def _num(v):
    return -0.0 if v == "-0" else float(v)


def _build_variant(tmp_path, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"the step {old!r} must occur once in the oracle"
    text = text.replace(old, new)
    text = text.replace("/* ---------------------------------------------------------- block quantizers */",
                        EXACT_ENCODER + "\n/* block quantizers */")
    src = tmp_path / "oracle_variant.c"
    src.write_text(text)
    lib = tmp_path / "liboracle_variant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-w", "-o", str(lib), str(src), "-lm"], check=True)
    L = ctypes.CDLL(str(lib))
    u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
    u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    L.oracle_prep_variant.restype = ci
    L.oracle_prep_variant.argtypes = [u16p, i64, i64, i64, ci, ci, ci, ci, u8p, u8p, vp, u8p, u8p, vp, vp, vp,
                                      vp]
    return L


def _outputs(L, ex):
    x = np.array([_num(v) for v in ex["x"]], np.float32)[None, :]
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x)
    K = x.shape[1]
    nv = ex["fmt"] == "nvfp4"
    bc = np.zeros((1, K // 2), np.uint8)
    bs = np.zeros((1, K // (16 if nv else 32)), np.uint8)
    rc = np.zeros_like(bc)
    rs = np.zeros_like(bs)
    bt = np.ones(1, np.float32)
    rt = np.ones(1, np.float32)
    resid = np.zeros((1, K), np.float32)
    mask = np.zeros((1, K // 8), np.uint8)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rcode = L.oracle_prep_variant(xb, 1, K, K, ex["n"], ex["m"], 1 if nv else 0, 0, bc, bs,
                                  ptr(bt) if nv else None, rc, rs, ptr(rt) if nv else None, ptr(mask), None,
                                  ptr(resid))
    assert rcode == 0

    def unpack(p):
        out = np.empty(K, np.uint8)
        out[0::2] = p[0] & 15
        out[1::2] = p[0] >> 4
        return out.tolist()

    want_r = np.array([_num(v) for v in ex["residual"]], np.float32)
    out = {
        "mask_bytes": mask[0].tolist() == ex["mask_bytes"],
        "backbone_codes": unpack(bc) == ex["backbone_codes"],
        "backbone_scales": bs[0].tolist() == ex["backbone_scales"],
        "residual_codes": unpack(rc) == ex["residual_codes"],
        "residual": np.array_equal(resid[0].view(np.uint32), want_r.view(np.uint32)),
    }
    if "residual_scales" in ex:
        out["residual_scales"] = rs[0].tolist() == ex["residual_scales"]
    if nv:
        out["tensor_scales"] = bt[0] == ex["backbone_tensor_scale"] and rt[0] == ex["residual_tensor_scale"]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
def test_unmodified_copy_reproduces_every_nv_example(tmp_path):
    L = _build_variant(tmp_path, "  float q = amax / six_s;", "  float q = amax / six_s;")
    for ex in _nv_examples():
        assert all(_outputs(L, ex).values()), ex["name"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_nv_examples_catch_a_deviation_from_r5(tmp_path, name, old, new):
    L = _build_variant(tmp_path, old, new)
    failed = {ex["name"]: [k for k, ok in _outputs(L, ex).items() if not ok] for ex in _nv_examples()}
    assert any(failed.values()), f"no worked example detects: {name}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
def test_unmodified_copy_reproduces_every_mx_example(tmp_path):
    L = _build_variant(tmp_path, "  int e = (e2 - 1) - 2;", "  int e = (e2 - 1) - 2;")
    for ex in _examples("mxfp4"):
        assert all(_outputs(L, ex).values()), ex["name"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
@pytest.mark.parametrize("name,old,new", MX_MUTATIONS, ids=[m[0] for m in MX_MUTATIONS])
def test_mx_examples_catch_a_deviation(tmp_path, name, old, new):
    L = _build_variant(tmp_path, old, new)
    failed = {ex["name"]: [k for k, ok in _outputs(L, ex).items() if not ok] for ex in _examples("mxfp4")}
    assert any(failed.values()), f"no worked example detects: {name}"


# Deviations from reading R7 (Y = Bhat W^T + Rhat W^T, exact products summed in fp64;
# SharQ, abstract: a sparse FP4 GEMM over the backbone and a dense FP4 GEMM over the
# residual share one weight payload and their products are summed), each caught by
# the exact-rational GEMM pin: Y computed from the payloads' values with Fractions.
GEMM_MUTATIONS = [
    ("residual product dropped", "      y[r * N + o] = yb + yr;", "      y[r * N + o] = yb; (void)yr;"),
    ("backbone product dropped", "      y[r * N + o] = yb + yr;", "      y[r * N + o] = yr; (void)yb;"),
    ("weight read transposed", "      const double* w = wd + o * K;", "      const double* w = wd + o;"),
    ("fp32 accumulation", "      double yb = 0.0, yr = 0.0;", "      float yb = 0.0f, yr = 0.0f;"),
    ("scale bias 128", "      out[i * K + k] = fmt == ORACLE_MXFP4 ? ldexp(v, (int)s - 127)",
     "      out[i * K + k] = fmt == ORACLE_MXFP4 ? ldexp(v, (int)s - 128)"),
]

_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
         Fraction(6)]


def _exact_mx_rows(codes, scales, K):
    rows = []
    for i in range(codes.shape[0]):
        row = []
        for k in range(K):
            c = (codes[i, k // 2] >> (4 * (k & 1))) & 15
            v = -_E2M1[c & 7] if c & 8 else _E2M1[c & 7]
            row.append(v * Fraction(2) ** (int(scales[i, k // 32]) - 127))
        rows.append(row)
    return rows


def _linear_variant(L, bb, rr, w, M, N, K):
    u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i64, f32 = ctypes.c_int64, ctypes.c_float
    L.oracle_linear.restype = ctypes.c_int
    L.oracle_linear.argtypes = [u8p, u8p, f32, u8p, u8p, f32, i64, u8p, u8p, f32, i64, i64, ctypes.c_int,
                                ctypes.c_void_p, i64, f64p]
    y = np.zeros((M, N), np.float64)
    assert L.oracle_linear(bb.codes, bb.scales, 1.0, rr.codes, rr.scales, 1.0, M, w.codes, w.scales, 1.0, N, K,
                           0, None, M, y) == 0
    return y


def _matches_exact(y, bb, rr, w, K):
    B, R, W = (_exact_mx_rows(p.codes, p.scales, K) for p in (bb, rr, w))
    for i in range(len(B)):
        for o in range(len(W)):
            exact = sum(B[i][k] * W[o][k] for k in range(K)) + sum(R[i][k] * W[o][k] for k in range(K))
            mag = sum(abs(B[i][k] * W[o][k]) + abs(R[i][k] * W[o][k]) for k in range(K))
            if abs(Fraction(y[i, o]) - exact) > Fraction(2 * K + 2) * Fraction(2) ** -53 * mag:
                return False
    return True


def _gemm_case():
    import oracle
    from activation_sparsity_fp4_sharq_amd.workloads import make_activation
    M, N, K = 3, 5, 96
    rng = np.random.default_rng(7)
    x = bf16_bits_to_f32(make_activation(rng, M, K, "normal", n_out=2, out_scale=20.0))
    # blocks 2^14 apart, so partial sums need more than fp32's 24 bits
    x = x * np.repeat(2.0 ** (14 * np.arange(K // 32)), 32)[None, :].astype(np.float32)
    wb = f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    bb, rr, _ = oracle.prep(f32_to_bf16_bits(x), 2, 4)
    return bb, rr, oracle.quantize(wb), M, N, K


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
def test_unmodified_copy_meets_the_exact_gemm(tmp_path):
    bb, rr, w, M, N, K = _gemm_case()
    L = _build_variant(tmp_path, "      y[r * N + o] = yb + yr;", "      y[r * N + o] = yb + yr;")
    assert _matches_exact(_linear_variant(L, bb, rr, w, M, N, K), bb, rr, w, K)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
@pytest.mark.parametrize("name,old,new", GEMM_MUTATIONS, ids=[m[0] for m in GEMM_MUTATIONS])
def test_exact_gemm_catches_a_deviation(tmp_path, name, old, new):
    bb, rr, w, M, N, K = _gemm_case()
    L = _build_variant(tmp_path, old, new)
    assert not _matches_exact(_linear_variant(L, bb, rr, w, M, N, K), bb, rr, w, K), f"not detected: {name}"


# Deviations from reading R9 (RMS normalization folded into the preparation) and R14 (the
# MLP block's SwiGLU), each planted in a copy of the oracle, which then serves the pins of
# tests/test_oracle_pins.py (through the oracle module, its library swapped for the copy's):
# at least one pin must fail.  Not caught, because they never reach the path's output h:
# R14's exponential evaluated by another correct method -- glibc's expf changes the fp32 SiLU
# of 124 bf16 gates in [-60, 60], a degree-6 instead of a degree-7 polynomial of 174 -- gives
# the same h for every bf16 up value in [2^-7, 2^8) (searched exhaustively), and both stay
# within the 4-ulp bound of the fp64 SiLU that the pins check.  An exponential one fp32 ulp
# off the reading's where that does reach h is caught by the hand-worked SwiGLU example.
R9_MUTATIONS = [
    ("mean over K + 1", "    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));",
     "    const float r = (float)(1.0 / sqrt(ss / (double)(K + 1) + (double)eps));"),
    ("eps outside the root", "    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));",
     "    const float r = (float)(1.0 / (sqrt(ss / (double)K) + (double)eps));"),
    ("r in fp32", "    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));",
     "    const float r = 1.0f / sqrtf((float)(ss / (double)K) + eps);"),
    ("gain applied first", "      const float t = bf16_to_f32(x[i * ldx + k]) * r;\n      const float u = t * bf16_to_f32(g[k]);",
     "      const float t = bf16_to_f32(x[i * ldx + k]) * bf16_to_f32(g[k]);\n      const float u = t * r;"),
    ("r and gain in one product", "      const float t = bf16_to_f32(x[i * ldx + k]) * r;\n      const float u = t * bf16_to_f32(g[k]);",
     "      const float u = bf16_to_f32(x[i * ldx + k]) * (r * bf16_to_f32(g[k]));"),
    ("sum of squares left to right", "  for (int64_t w = p; w > 1; w /= 2)\n    for (int64_t j = 0; j < w / 2; ++j) v[j] = v[2 * j] + v[2 * j + 1];",
     "  for (int64_t j = 1; j < p; ++j) v[0] = v[0] + v[j];"),
    ("bf16 by truncation", "      y[i * K + k] = f32_to_bf16(u);",
     "      { union { float f; uint32_t b; } c; c.f = u; y[i * K + k] = (uint16_t)(c.b >> 16); }"),
]
R14_MUTATIONS = [
    ("gate and up swapped", "      h[i * I + k] = f32_to_bf16(oracle_silu(g) * u);",
     "      h[i * I + k] = f32_to_bf16(oracle_silu(u) * g);"),
    ("logistic without the 1", "  const float d = 1.0f + swiglu_exp_neg(g);", "  const float d = swiglu_exp_neg(g);"),
    ("ln 2 without its low part", "  const float r = (t - n * ln2_hi) - n * ln2_lo;",
     "  const float r = t - n * ln2_hi; (void)ln2_lo;"),
    ("exponent clamped at 80", "  if (t > 150.0f) t = 150.0f;", "  if (t > 80.0f) t = 80.0f;"),
    ("exponential one ulp high", "  return ldexpf(p, (int)n);", "  return nextafterf(ldexpf(p, (int)n), INFINITY);"),
]


def _pins_fail(tmp_path, old, new, calls):
    import oracle
    _build_variant(tmp_path, old, new)  # writes liboracle_variant.so
    saved = (oracle._lib, oracle._LIB_PATH)
    oracle._lib, oracle._LIB_PATH = None, str(tmp_path / "liboracle_variant.so")
    try:
        oracle.lib()
        failed = []
        for name, call in calls:
            try:
                call()
            except AssertionError:
                failed.append(name)
        return failed
    finally:
        oracle._lib, oracle._LIB_PATH = saved


def _r9_pins():
    import test_oracle_pins as p
    return [("closed forms", p.test_rmsnorm_closed_forms),
            ("unit mean square", p.test_rmsnorm_unit_mean_square_with_unit_gain),
            ("power-of-two input scaling", lambda: p.test_rmsnorm_invariant_under_power_of_two_input_scaling(3)),
            ("power-of-two gain", lambda: p.test_rmsnorm_gain_power_of_two_is_exact(2)),
            ("small-integer sums", lambda: p.test_row_sumsq_exact_on_small_integers(1024)),
            ("run-tree order", p.test_row_sumsq_order_is_the_run_tree),
            ("hand-worked rounding sequence", p.test_rmsnorm_hand_worked_rounding_sequence)]


def _r14_pins():
    import test_oracle_pins as p
    return [("closed forms", p.test_silu_closed_forms),
            ("error bound over every bf16", p.test_silu_matches_the_mathematics_over_every_bf16_in_range),
            ("layout and special inputs", p.test_swiglu_layout_and_special_inputs),
            ("hand-worked example", p.test_swiglu_hand_worked_example)]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
def test_unmodified_copy_meets_the_r9_and_r14_pins(tmp_path):
    old = "  if (t > 150.0f) t = 150.0f;"
    assert _pins_fail(tmp_path, old, old, _r9_pins() + _r14_pins()) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
@pytest.mark.parametrize("name,old,new", R9_MUTATIONS, ids=[m[0] for m in R9_MUTATIONS])
def test_r9_pins_catch_a_deviation(tmp_path, name, old, new):
    assert _pins_fail(tmp_path, old, new, _r9_pins()), f"no R9 pin detects: {name}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the oracle variants")
@pytest.mark.parametrize("name,old,new", R14_MUTATIONS, ids=[m[0] for m in R14_MUTATIONS])
def test_r14_pins_catch_a_deviation(tmp_path, name, old, new):
    assert _pins_fail(tmp_path, old, new, _r14_pins()), f"no R14 pin detects: {name}"
