"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: masks, FP4 codes, scale bytes and tensor scales bit-exact; GEMM output within
max-norm relative error 2e-3 of the oracle's fp64 result (fp32 output), and for the
bf16 output every element within one bf16 ulp of the oracle rounded to bf16 plus a
Frobenius relative error <= 2e-3.  Inputs come from the seeded generators only.
"""
import numpy as np
import pytest
import torch

import layout_ref
import oracle
from activation_sparsity_fp4_sharq_amd import sharq
from activation_sparsity_fp4_sharq_amd.workloads import (WORKLOADS, adversarial_activation,
                                                          f32_to_bf16_bits, make_inputs, make_shape)

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = torch.device("cuda:0")


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_rowmajor(p):
    """A device payload as row-major numpy arrays; tiled payloads are un-tiled on the host
    by the test's own reference of the layout (not by the library)."""
    if p.layout == sharq.TILED:
        ct, st = p.raw_host()
        assert layout_ref.padding_is_zero(ct, st, p.rows, p.K), "tiled padding not zero"
        c, s = layout_ref.untile(ct, st, p.rows, p.K)
        return c, s, 1.0
    return p.to_host()


def assert_payload_equal(got, want, what):
    gc, gs, gt = host_rowmajor(got)
    assert gc.shape == want.codes.shape and gs.shape == want.scales.shape, what
    bad = np.nonzero(gc != want.codes)
    assert bad[0].size == 0, f"{what}: {bad[0].size} code bytes differ, first at {bad[0][0]},{bad[1][0]}"
    bad = np.nonzero(gs != want.scales)
    assert bad[0].size == 0, f"{what}: {bad[0].size} scale bytes differ, first at {bad[0][0]},{bad[1][0]}"
    if got.fmt == sharq.NVFP4:
        assert np.float32(gt) == np.float32(want.tscale), f"{what}: tensor scale {gt} != {want.tscale}"


def check_prep(xb, n, m, fmt, ldx_pad=0, layout=None):
    M, K = xb.shape
    if ldx_pad:
        wide = np.zeros((M, K + ldx_pad), np.uint16)
        wide[:, :K] = xb
        x = to_dev(wide)[:, :K]
    else:
        x = to_dev(xb)
    bb, rr, mask = sharq.prep(x, n, m, fmt, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    ob, orr, omask = oracle.prep(xb, n, m, fmt)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")
    return ob, orr


def rel_maxnorm(y, yref):
    den = np.abs(yref).max()
    return np.abs(y - yref).max() / (den if den > 0 else 1.0)


def bf16_ulp_check(ybf, yref):
    """Every bf16 output within one ulp of the oracle value rounded to bf16."""
    want = f32_to_bf16_bits(yref.astype(np.float32)).astype(np.int32)
    got = ybf.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.int32)
    # bf16 bits are sign-magnitude; compare as ordered integers
    def ordered(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(ordered(got) - ordered(want)).max()


def bf16_bound_check(ybf, yref, abssum, K):
    """Every bf16 output within one bf16 ulp of the exact value plus the fp32 summation
    bound: the kernels form every product exactly and sum K of them (two paths) in fp32,
    then apply at most 4 rounded scale operations, so |y32 - exact| <= (K + 4) 2^-24
    sum|terms| (sum|terms| = the same GEMM over absolute values); rounding y32 to bf16
    adds at most half an ulp.  Where the sum cancels (|exact| far below sum|terms|) the
    first term alone would be unattainable.  Returns the worst |error| / allowance."""
    got = ybf.float().cpu().numpy().astype(np.float64)
    mag = np.maximum(np.abs(yref), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    allowed = ulp + (K + 4) * 2.0 ** -24 * abssum
    return float((np.abs(got - yref) / allowed).max())


def abs_linear(ob, orr, ow, fmt):
    """sum over k of |Bhat w| + |Rhat w| for every output, in fp64 from the oracle's exact values."""
    wa = np.abs(oracle.dequant(ow, fmt))
    return np.abs(oracle.dequant(ob, fmt)) @ wa.T + np.abs(oracle.dequant(orr, fmt)) @ wa.T


# ------------------------------------------------------------------ prep parity

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_prep_workloads_full_size(name):
    w = WORKLOADS[name]
    print(f"[prep] {name} M={w.M} K={w.K} {w.n}:{w.m} fmt={w.fmt}", flush=True)
    xb, _ = make_inputs(w, with_weight=False)
    check_prep(xb, w.n, w.m, w.fmt)


FMT_LAYOUTS = [(sharq.MXFP4, sharq.TILED), (sharq.MXFP4, sharq.ROWMAJOR), (sharq.NVFP4, sharq.ROWMAJOR)]
FL_IDS = ["mx-tiled", "mx-rowmajor", "nv-rowmajor"]


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (17, 96), (100, 160), (300, 512), (65, 1056)])
def test_prep_shapes(fmt, layout, n, m, M, K):
    print(f"[prep] shape M={M} K={K} {n}:{m} fmt={fmt} layout={layout}", flush=True)
    xb, _ = make_shape(M, 8, K, seed=M * 131 + K, dist="student_t3", token_sigma=0.5)
    check_prep(xb, n, m, fmt, layout=layout)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_prep_adversarial(fmt, layout, n, m):
    print(f"[prep] adversarial {n}:{m} fmt={fmt} layout={layout}", flush=True)
    xb = adversarial_activation(96, 256, seed=3)
    check_prep(xb, n, m, fmt, layout=layout)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
def test_prep_strided_rows(fmt, layout):
    print(f"[prep] strided ldx fmt={fmt} layout={layout}", flush=True)
    xb, _ = make_shape(37, 8, 256, seed=5)
    check_prep(xb, 2, 4, fmt, ldx_pad=24, layout=layout)


@pytest.mark.parametrize("fmt", [sharq.MXFP4, sharq.NVFP4])
def test_prep_empty_and_zero(fmt):
    print(f"[prep] empty/zero fmt={fmt}", flush=True)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    bb, rr, _ = sharq.prep(x, 2, 4, fmt)
    torch.cuda.synchronize()
    assert bb.codes.numel() == 0 and bb.rows == 0
    if fmt == sharq.NVFP4:
        assert bb.tensor_scale[0].item() == 1.0 and rr.tensor_scale[0].item() == 1.0
    check_prep(np.zeros((5, 64), np.uint16), 2, 4, fmt)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("rows,K", [(512, 512), (77, 96), (14336, 4096)])
def test_quantize_weight(fmt, layout, rows, K):
    print(f"[quant] rows={rows} K={K} fmt={fmt} layout={layout}", flush=True)
    rng = np.random.default_rng(rows + K)
    wb = f32_to_bf16_bits(rng.normal(0, 0.02, (rows, K)).astype(np.float32))
    got = sharq.quantize(to_dev(wb), fmt, layout=layout)
    torch.cuda.synchronize()
    assert_payload_equal(got, oracle.quantize(wb, fmt), "weight")


def test_prep_deterministic_and_no_overrun():
    """Two runs are bitwise identical; bytes past the outputs stay untouched."""
    print("[prep] determinism/guard", flush=True)
    xb, _ = make_shape(123, 8, 352, seed=9)
    x = to_dev(xb)
    M, K = xb.shape
    outs = []
    for _ in range(2):
        big_c = torch.full((M * K // 2 + 4096,), 0xAA, dtype=torch.uint8, device=DEV)
        big_s = torch.full((M * K // 32 + 4096,), 0xAA, dtype=torch.uint8, device=DEV)
        big_rc = torch.full_like(big_c, 0xAA)
        big_rs = torch.full_like(big_s, 0xAA)
        ts = torch.zeros(4, dtype=torch.float32, device=DEV)
        bb = sharq.Payload(big_c[:M * K // 2], big_s[:M * K // 32], ts, sharq.MXFP4, sharq.ROWMAJOR, M, K)
        rr = sharq.Payload(big_rc[:M * K // 2], big_rs[:M * K // 32], ts, sharq.MXFP4, sharq.ROWMAJOR, M, K)
        sharq.prep(x, 2, 4, sharq.MXFP4, out=(bb, rr))
        torch.cuda.synchronize()
        for big, n in ((big_c, M * K // 2), (big_s, M * K // 32), (big_rc, M * K // 2), (big_rs, M * K // 32)):
            assert torch.all(big[n:] == 0xAA), "write past the end of an output"
        outs.append([t.cpu().numpy().copy() for t in (big_c, big_s, big_rc, big_rs)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ GEMM parity

def run_linear(xb, wb, n, m, fmt, layout=None):
    x, wt = to_dev(xb), to_dev(wb)
    weight = sharq.quantize(wt, fmt, layout=layout)
    bb, rr, _ = sharq.prep(x, n, m, fmt, layout=layout)
    y32 = sharq.linear(bb, rr, weight, sharq.OUT_FP32)
    y16 = sharq.linear(bb, rr, weight, sharq.OUT_BF16)
    torch.cuda.synchronize()
    return weight, bb, rr, y32, y16


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 512, 512), (37, 70, 96), (300, 260, 160),
                                   (257, 513, 1056), (64, 256, 2048), (520, 300, 384),
                                   (32, 1000, 4224), (7, 96, 640), (33, 96, 640), (20, 200, 384),
                                   (2000, 4000, 512)])
def test_linear_small_full_compare(fmt, layout, M, N, K):
    print(f"[linear] M={M} N={N} K={K} fmt={fmt} layout={layout}", flush=True)
    xb, wb = make_shape(M, N, K, seed=M + N + K, dist="laplace", token_sigma=0.3)
    weight, bb, rr, y32, y16 = run_linear(xb, wb, 2, 4, fmt, layout)
    ob, orr, _ = oracle.prep(xb, 2, 4, fmt)
    ow = oracle.quantize(wb, fmt)
    assert_payload_equal(weight, ow, "weight")
    yref = oracle.linear(ob, orr, ow, fmt)
    err = rel_maxnorm(y32.cpu().numpy().astype(np.float64), yref)
    assert err <= TOL, f"fp32 output max-norm rel err {err}"
    assert bf16_bound_check(y16, yref, abs_linear(ob, orr, ow, fmt), K) <= 1.0
    # bf16 rounding alone is up to 2^-8 relative per element, so the Frobenius bound is
    # only meaningful over many outputs; the one-ulp check above covers small cases
    if y16.numel() >= 1024:
        fro = np.linalg.norm(y16.float().cpu().numpy() - yref) / max(np.linalg.norm(yref), 1e-300)
        assert fro <= TOL


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 512, 512), (37, 70, 96), (257, 513, 1056),
                                   (64, 256, 2048), (520, 300, 384), (33, 96, 640)])
def test_linear_dense_matches_oracle(fmt, layout, M, N, K):
    """Plain FP4 linear (the SharQ kernels with the backbone path off)."""
    print(f"[linear_dense] M={M} N={N} K={K} fmt={fmt} layout={layout}", flush=True)
    xb, wb = make_shape(M, N, K, seed=3 * M + N + K, dist="laplace", token_sigma=0.3)
    x, wt = to_dev(xb), to_dev(wb)
    weight = sharq.quantize(wt, fmt, layout=layout)
    a = sharq.quantize(x, fmt, layout=layout)
    y32 = sharq.linear_dense(a, weight, sharq.OUT_FP32)
    y16 = sharq.linear_dense(a, weight, sharq.OUT_BF16)
    torch.cuda.synchronize()
    oa, ow = oracle.quantize(xb, fmt), oracle.quantize(wb, fmt)
    assert_payload_equal(a, oa, "activation")
    assert_payload_equal(weight, ow, "weight")
    yref = oracle.linear_dense(oa, ow, fmt)
    err = rel_maxnorm(y32.cpu().numpy().astype(np.float64), yref)
    assert err <= TOL, f"fp32 output max-norm rel err {err}"
    assert bf16_ulp_check(y16, yref) <= 1


@pytest.mark.parametrize("name", ["prefill", "decode", "mlp_down_nvfp4", "dit"])
def test_linear_dense_workloads_sampled_rows(name):
    """Plain FP4 linear at the full workload shapes (the comparison point of the benchmark)."""
    w = WORKLOADS[name]
    print(f"[linear_dense] {name} M={w.M} N={w.N} K={w.K} fmt={w.fmt}", flush=True)
    xb, wb = make_inputs(w)
    x, wt = to_dev(xb), to_dev(wb)
    weight = sharq.quantize(wt, w.fmt)
    a = sharq.quantize(x, w.fmt)
    y32 = sharq.linear_dense(a, weight, sharq.OUT_FP32)
    torch.cuda.synchronize()
    oa, ow = oracle.quantize(xb, w.fmt), oracle.quantize(wb, w.fmt)
    assert_payload_equal(a, oa, "activation")
    rows = np.unique(np.concatenate([np.arange(min(8, w.M)), np.arange(max(0, w.M - 8), w.M),
                                     np.linspace(0, w.M - 1, 16).astype(np.int64)]))
    yref = oracle.linear_dense(oa, ow, w.fmt, rows=rows)
    err = rel_maxnorm(y32.cpu().numpy()[rows].astype(np.float64), yref)
    assert err <= TOL, f"{name}: fp32 output max-norm rel err {err}"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_linear_workloads_sampled_rows(name):
    """Full-size shapes in the benchmark's launch configuration; the oracle computes
    a sample of rows (first, last, and a spread in between) over all N columns."""
    w = WORKLOADS[name]
    print(f"[linear] {name} M={w.M} N={w.N} K={w.K} fmt={w.fmt}", flush=True)
    xb, wb = make_inputs(w)
    x, wt = to_dev(xb), to_dev(wb)
    weight = sharq.quantize(wt, w.fmt)
    y32, (bb, rr) = sharq.forward(x, weight, w.n, w.m, out_dtype=sharq.OUT_FP32)
    y16, _ = sharq.forward(x, weight, w.n, w.m, out_dtype=sharq.OUT_BF16, bufs=(bb, rr))
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(xb, w.n, w.m, w.fmt)
    ow = oracle.quantize(wb, w.fmt)
    assert_payload_equal(weight, ow, "weight")
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")
    rows = np.unique(np.concatenate([np.arange(min(8, w.M)), np.arange(max(0, w.M - 8), w.M),
                                     np.linspace(0, w.M - 1, 16).astype(np.int64)]))
    yref = oracle.linear(ob, orr, ow, w.fmt, rows=rows)
    y = y32.cpu().numpy()[rows].astype(np.float64)
    err = rel_maxnorm(y, yref)
    assert err <= TOL, f"{name}: fp32 output max-norm rel err {err}"
    assert bf16_ulp_check(y16[torch.from_numpy(rows).to(DEV)], yref) <= 1


def test_linear_deterministic_and_guarded():
    print("[linear] determinism/guard", flush=True)
    M, N, K = 300, 260, 256
    xb, wb = make_shape(M, N, K, seed=77)
    x, wt = to_dev(xb), to_dev(wb)
    weight = sharq.quantize(wt, sharq.MXFP4)
    bb, rr, _ = sharq.prep(x, 2, 4)
    res = []
    for _ in range(2):
        ld = N + 8
        big = torch.full(((M + 2) * ld,), float("nan"), dtype=torch.float32, device=DEV)
        y = big[:M * ld].view(M, ld)
        sharq.linear(bb, rr, weight, sharq.OUT_FP32, y=y)
        torch.cuda.synchronize()
        out = big.cpu().numpy()
        assert np.all(np.isnan(out[M * ld:])), "write past the output"
        assert np.all(np.isnan(out[:M * ld].reshape(M, ld)[:, N:])), "write into the ld padding"
        res.append(out[:M * ld].reshape(M, ld)[:, :N].copy())
    assert np.array_equal(res[0], res[1])


@pytest.mark.parametrize("fmt", [sharq.MXFP4, sharq.NVFP4], ids=["mx", "nv"])
@pytest.mark.parametrize("M,N,K", [(2040, 4090, 128), (1930, 3850, 64)])
def test_linear_large_tiles_strided_output(fmt, M, N, K):
    """The large-M kernels' bf16 epilogues (LDS-staged 16-byte row stores where a wave's
    tile lies inside Y and rows are 16-byte aligned, element stores elsewhere) with a row
    pitch padded to a multiple of 8, with an odd pitch, and with ragged M and N: the same
    values as the contiguous output, nothing written past a row's N columns or past Y.
    (1930 x 3850 leaves whole waves of the last row and column tiles outside Y; K = 64 is
    a single K-step.)"""
    print(f"[linear] strided bf16 output M={M} N={N} K={K} fmt={fmt}", flush=True)
    xb, wb = make_shape(M, N, K, seed=91)
    weight = sharq.quantize(to_dev(wb), fmt)
    bb, rr, _ = sharq.prep(to_dev(xb), 2, 4, fmt)
    y16 = sharq.linear(bb, rr, weight, sharq.OUT_BF16)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(xb, 2, 4, fmt)
    ow = oracle.quantize(wb, fmt)
    assert bf16_bound_check(y16, oracle.linear(ob, orr, ow, fmt), abs_linear(ob, orr, ow, fmt), K) <= 1.0
    ref = y16.view(torch.int16).cpu().numpy()
    for ld in (N + 6, N + 3):
        big = torch.full(((M + 1) * ld,), -1, dtype=torch.int16, device=DEV)  # 0xFFFF: a bf16 NaN
        y = big.view(torch.bfloat16)[:M * ld].view(M, ld)[:, :N]  # row pitch ld
        sharq.linear(bb, rr, weight, sharq.OUT_BF16, y=y)
        torch.cuda.synchronize()
        out = big.cpu().numpy()
        assert np.all(out[M * ld:] == -1), f"ld={ld}: write past the output"
        rows = out[:M * ld].reshape(M, ld)
        assert np.all(rows[:, N:] == -1), f"ld={ld}: write into the row padding"
        assert np.array_equal(rows[:, :N], ref), f"ld={ld}: values differ from the contiguous output"


# ------------------------------------------------------------------ layouts

@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (300, 1056), (64, 4096)])
def test_convert_layout_matches_reference(rows, K):
    """sharq_convert_layout against the test's host reference of the tiled layout, both ways."""
    print(f"[layout] rows={rows} K={K}", flush=True)
    rng = np.random.default_rng(rows * 7 + K)
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, K // 32), dtype=np.uint8)
    rm = sharq.Payload(torch.from_numpy(codes.reshape(-1)).to(DEV), torch.from_numpy(scales.reshape(-1)).to(DEV),
                       torch.ones(4, device=DEV), sharq.MXFP4, sharq.ROWMAJOR, rows, K)
    t = rm.convert(sharq.TILED)
    back = t.convert(sharq.ROWMAJOR)
    torch.cuda.synchronize()
    ct, st = layout_ref.tile(codes, scales)
    gct, gst = t.raw_host()
    assert np.array_equal(gct, ct) and np.array_equal(gst, st)
    bc, bs, _ = back.to_host()
    assert np.array_equal(bc, codes) and np.array_equal(bs, scales)


def test_linear_rejects_mixed_layouts():
    xb, wb = make_shape(64, 64, 128, seed=1)
    x, wt = to_dev(xb), to_dev(wb)
    w_rm = sharq.quantize(wt, sharq.MXFP4, layout=sharq.ROWMAJOR)
    bb, rr, _ = sharq.prep(x, 2, 4, sharq.MXFP4, layout=sharq.TILED)
    with pytest.raises(sharq.SharqError) as e:
        sharq.linear(bb, rr, w_rm)
    assert e.value.status == 4


# ------------------------------------------------------------ RMSNorm folded into the prep

def _gain(K, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.normal(1.0, 0.25, K).astype(np.float32))


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("M,K,ldx_pad", [(1, 64, 0), (37, 352, 0), (300, 1024, 64), (128, 4096, 0)])
def test_prep_rmsnorm_matches_oracle(fmt, layout, n, m, M, K, ldx_pad):
    """sharq_prep_rmsnorm == oracle.prep(oracle.rmsnorm(x)): masks, codes, scale bytes
    and tensor scales bit for bit."""
    print(f"[prep_rmsnorm] fmt={fmt} layout={layout} {n}:{m} M={M} K={K} pad={ldx_pad}", flush=True)
    xb, _ = make_shape(M, 8, K, seed=M * 7 + K, dist="student_t3", token_sigma=0.8)
    g = _gain(K, K)
    eps = 1e-5
    if ldx_pad:
        wide = np.zeros((M, K + ldx_pad), np.uint16)
        wide[:, :K] = xb
        x = to_dev(wide)[:, :K]
    else:
        x = to_dev(xb)
    bb, rr, mask = sharq.prep_rmsnorm(x, to_dev(g), eps, n, m, fmt, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    yb, _ = oracle.rmsnorm(xb, g, eps)
    ob, orr, omask = oracle.prep(yb, n, m, fmt)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


def test_prep_rmsnorm_workload_full_size():
    """The prefill workload's activation through the normalized preparation."""
    w = WORKLOADS["prefill"]
    print("[prep_rmsnorm] prefill full size", flush=True)
    xb, _ = make_inputs(w, with_weight=False)
    g = _gain(w.K, 1)
    bb, rr, _ = sharq.prep_rmsnorm(to_dev(xb), to_dev(g), 1e-6, w.n, w.m, w.fmt)
    torch.cuda.synchronize()
    yb, _ = oracle.rmsnorm(xb, g, 1e-6)
    ob, orr, _ = oracle.prep(yb, w.n, w.m, w.fmt)
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


# ------------------------------------------------------------------ ablations and dequantization

ABLATIONS = [sharq.ABLATE_RESIDUAL_UNQUANTIZED, sharq.ABLATE_STATIC_MASK, sharq.ABLATE_NO_RESIDUAL]


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("variant", ABLATIONS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("M,K,ldx_pad", [(1, 64, 0), (37, 352, 0), (300, 1024, 64)])
def test_prep_ablation_matches_oracle(fmt, layout, variant, n, m, M, K, ldx_pad):
    print(f"[prep_ablation] variant={variant} {n}:{m} M={M} K={K} fmt={fmt} layout={layout}", flush=True)
    rng = np.random.default_rng(M * 7 + K + variant)
    from activation_sparsity_fp4_sharq_amd.workloads import make_activation
    xb = make_activation(rng, M, K, "laplace", n_out=max(1, K // 64), out_scale=20.0)
    if ldx_pad:
        wide = np.zeros((M, K + ldx_pad), np.uint16)
        wide[:, :K] = xb
        x = to_dev(wide)[:, :K]
    else:
        x = to_dev(xb)
    bb, rr, mask = sharq.prep_ablation(x, variant, n, m, fmt, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    ob, orr, omask = oracle.prep(xb, n, m, fmt, variant=variant)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


@pytest.mark.parametrize("variant", ABLATIONS)
def test_prep_ablation_full_size_prefill(variant):
    w = WORKLOADS["prefill"]
    print(f"[prep_ablation] prefill variant={variant}", flush=True)
    xb, _ = make_inputs(w)
    bb, rr, _ = sharq.prep_ablation(to_dev(xb), variant, w.n, w.m, w.fmt)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(xb, w.n, w.m, w.fmt, variant=variant)
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (300, 1056), (64, 4096)])
def test_dequantize_matches_oracle(fmt, layout, rows, K):
    if fmt == sharq.NVFP4 and K % 16:
        pytest.skip("not an NVFP4 shape")
    print(f"[dequantize] rows={rows} K={K} fmt={fmt} layout={layout}", flush=True)
    xb, _ = make_shape(rows, 8, K, seed=rows + K, dist="laplace", token_sigma=0.3)
    p = sharq.quantize(to_dev(xb), fmt, layout=layout)
    got = sharq.dequantize(p).cpu().numpy()
    torch.cuda.synchronize()
    want = oracle.dequant(oracle.quantize(xb, fmt), fmt).astype(np.float32)  # exact values, one rounding
    assert np.array_equal(got, want)


def test_clock_probe_reports_a_plausible_clock():
    print("[clock_probe]", flush=True)
    hz = sharq.clock_probe(20000)
    assert 0.5e9 < hz < 3.5e9, hz


# ------------------------------------------------------------------ SwiGLU-fused preparation

def _gate_up(M, I, pad, seed):
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, 3.0, (M, I)) * rng.lognormal(0.0, 0.5, (M, 1))
    u = rng.normal(0.0, 1.0, (M, I))
    gu = np.zeros((M, 2 * I + pad), np.uint16)
    gu[:, :I] = f32_to_bf16_bits(g.astype(np.float32))
    gu[:, I:2 * I] = f32_to_bf16_bits(u.astype(np.float32))
    return gu


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("M,I,pad", [(1, 64, 0), (37, 352, 16), (300, 1024, 0)])
def test_prep_swiglu_matches_oracle(fmt, layout, n, m, M, I, pad):
    print(f"[prep_swiglu] {n}:{m} M={M} I={I} pad={pad} fmt={fmt} layout={layout}", flush=True)
    gu = _gate_up(M, I, pad, seed=M + I + pad)
    bb, rr, mask = sharq.prep_swiglu(to_dev(gu), I, n, m, fmt, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    h = oracle.swiglu(gu, I)
    ob, orr, omask = oracle.prep(h, n, m, fmt)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


def test_prep_swiglu_full_size_mlp():
    """The MLP block's down-projection preparation at its full shape (M=2048, I=14336)."""
    print("[prep_swiglu] M=2048 I=14336", flush=True)
    M, I = 2048, 14336
    gu = _gate_up(M, I, 0, seed=5)
    bb, rr, _ = sharq.prep_swiglu(to_dev(gu), I, 2, 4, sharq.MXFP4, layout=sharq.TILED)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(oracle.swiglu(gu, I), 2, 4, sharq.MXFP4)
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


def test_mlp_block_chain_matches_oracle():
    """The MLP block (prep -> gate/up linear -> SwiGLU-fused prep -> down linear) stage by
    stage; each oracle stage takes the GPU's previous output, so what is unique is compared:
    payloads bit for bit, GEMM outputs within the tolerance."""
    from activation_sparsity_fp4_sharq_amd.workloads import MLP_BLOCKS, make_mlp_inputs
    b = MLP_BLOCKS["mlp_block_small"]
    print(f"[mlp_block] M={b.M} H={b.H} I={b.I}", flush=True)
    xb, wgub, wdb = make_mlp_inputs(b)
    wgu = sharq.quantize(to_dev(wgub), b.fmt)
    wd = sharq.quantize(to_dev(wdb), b.fmt)
    b1, r1, _ = sharq.prep(to_dev(xb), b.n, b.m, b.fmt)
    gu = sharq.linear(b1, r1, wgu, sharq.OUT_BF16)
    b2, r2, _ = sharq.prep_swiglu(gu, b.I, b.n, b.m, b.fmt)
    y32 = sharq.linear(b2, r2, wd, sharq.OUT_FP32)
    torch.cuda.synchronize()
    ob1, or1, _ = oracle.prep(xb, b.n, b.m, b.fmt)
    assert_payload_equal(b1, ob1, "backbone 1")
    assert_payload_equal(r1, or1, "residual 1")
    ref_gu = oracle.linear(ob1, or1, oracle.quantize(wgub, b.fmt), b.fmt)
    assert bf16_ulp_check(gu, ref_gu) <= 1
    gu_bits = gu.cpu().view(torch.int16).numpy().view(np.uint16)
    ob2, or2, _ = oracle.prep(oracle.swiglu(gu_bits, b.I), b.n, b.m, b.fmt)
    assert_payload_equal(b2, ob2, "backbone 2")
    assert_payload_equal(r2, or2, "residual 2")
    yref = oracle.linear(ob2, or2, oracle.quantize(wdb, b.fmt), b.fmt)
    err = rel_maxnorm(y32.cpu().numpy().astype(np.float64), yref)
    assert err <= TOL, err
