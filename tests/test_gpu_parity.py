"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: masks, FP4 codes, scale bytes and tensor scales bit-exact; GEMM output within
max-norm relative error 2e-3 of the oracle's fp64 result (fp32 output) and, element by
element, within the fp32 summation bound (2K + 4) 2^-24 sum|terms| of it; for the bf16
output every element within one bf16 ulp of the oracle plus that bound, and a Frobenius
relative error <= 2e-3.  Inputs come from the seeded generators only; the worked examples
of tests/golden/hand_examples.json are compared with their stored (hand-derived) values.
"""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import layout_ref
import oracle
from activation_sparsity_fp4_sharq_amd import sharq
from activation_sparsity_fp4_sharq_amd.workloads import (WORKLOADS, adversarial_activation, bf16_bits_to_f32,
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
    """sum over k of |Bhat w| + |Rhat w| for every output, in fp64 from the oracle's exact
    values (one product of the summed magnitudes: |Bhat| + |Rhat| against |W|)."""
    wa = np.abs(oracle.dequant(ow, fmt))
    a = np.abs(oracle.dequant(ob, fmt))
    a += np.abs(oracle.dequant(orr, fmt))
    return a @ wa.T


def fp32_bound_check(y32, yref, abssum, K):
    """Every fp32 output within the summation bound of the exact value: the kernels form
    each product of two FP4 values and their scales exactly and add the 2K products of the
    two paths in fp32 (in any order), then apply at most 4 rounded scale operations, so
    |y32 - exact| <= (2K + 4) 2^-24 sum|terms| to first order.  A wrong or missing product
    anywhere -- also in an output of small magnitude -- exceeds it.  Returns the worst
    |error| / allowance."""
    got = y32.cpu().numpy().astype(np.float64) if torch.is_tensor(y32) else y32
    allowed = (2 * K + 4) * 2.0 ** -24 * abssum + 2.0 ** -149
    return float((np.abs(got - yref) / allowed).max())


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
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_prep_signed_zeros_beside_ordinary_values(fmt, layout, n, m):
    """+0 and -0 among ordinary values, so that zeros sit in blocks with a nonzero scale:
    a -0 that is kept, or dropped and so carried into the residual, codes as 0x8 (E2M1
    keeps the sign of a zero quotient), a +0 as 0x0."""
    print(f"[prep] signed zeros {n}:{m} fmt={fmt} layout={layout}", flush=True)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    z = rng.random((64, 256))
    x[z < 0.3] = -0.0
    x[(z >= 0.3) & (z < 0.45)] = 0.0
    xb = f32_to_bf16_bits(x)
    check_prep(xb, n, m, fmt, layout=layout)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_prep_every_bf16_value(fmt, layout, n, m):
    """Every finite bf16 pattern once, shuffled over 512 rows x 128 columns: each block
    mixes magnitudes from subnormals to the bf16 maximum (which also sets NVFP4's tensor
    scales), signed zeros included."""
    print(f"[prep] every bf16 value {n}:{m} fmt={fmt} layout={layout}", flush=True)
    rng = np.random.default_rng(13)
    xb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xb[(xb & 0x7F80) == 0x7F80] = 0  # infinities and NaN are not part of the contract
    rng.shuffle(xb)
    check_prep(xb.reshape(512, 128), n, m, fmt, layout=layout)


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
def test_prep_strided_rows(fmt, layout):
    print(f"[prep] strided ldx fmt={fmt} layout={layout}", flush=True)
    xb, _ = make_shape(37, 8, 256, seed=5)
    check_prep(xb, 2, 4, fmt, ldx_pad=24, layout=layout)


def _hand_examples():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")
    with open(path) as f:
        return json.load(f)["examples"]


def _layouts_of(ex):
    return [sharq.TILED, sharq.ROWMAJOR] if ex["fmt"] == "mxfp4" else [sharq.ROWMAJOR]


@pytest.mark.parametrize("ex", _hand_examples(), ids=lambda e: e["name"])
def test_prep_hand_examples(ex):
    """The worked examples' stored, hand-derived values (not the oracle's): mask bytes,
    codes, scale bytes and tensor scales of the GPU preparation."""
    x = np.array([-0.0 if v == "-0" else float(v) for v in ex["x"]], np.float32)[None, :]
    xb = f32_to_bf16_bits(x)
    K = x.shape[1]
    fmt = sharq.MXFP4 if ex["fmt"] == "mxfp4" else sharq.NVFP4
    for layout in _layouts_of(ex):
        print(f"[prep] hand example {ex['name']} layout={layout}", flush=True)
        bb, rr, mask = sharq.prep(to_dev(xb), ex["n"], ex["m"], fmt, want_mask=True, layout=layout)
        torch.cuda.synchronize()
        assert mask.cpu().numpy()[0].tolist() == ex["mask_bytes"]
        for p, pre in ((bb, "backbone"), (rr, "residual")):
            c, sc, ts = host_rowmajor(p)
            codes = np.empty(K, np.uint8)
            codes[0::2] = c[0] & 15
            codes[1::2] = c[0] >> 4
            assert codes.tolist() == ex[pre + "_codes"], pre
            assert sc[0].tolist() == ex[pre + "_scales"], pre
            if fmt == sharq.NVFP4:
                assert np.float32(ts) == np.float32(ex[pre + "_tensor_scale"]), pre


@pytest.mark.parametrize("M,K,n,m", [(2048, 14336, 2, 4), (2049, 14336, 2, 4), (4096, 8192, 4, 8), (1, 16, 2, 4),
                                     (3000, 96, 2, 4)])
def test_prep_nvfp4_full_sizes_reuse_workspace(M, K, n, m):
    """The NVFP4 preparation at and around the MLP down-projection size, with both
    patterns and tiny and ragged shapes: bit-exact, and a second call with the same
    workspace (first filled with 0xA5) reproduces every byte -- each call writes every
    workspace word it reads before reading it."""
    print(f"[prep] nvfp4 M={M} K={K} {n}:{m}", flush=True)
    xb, _ = make_shape(M, 8, K, seed=M + K, dist="laplace", out_frac=0.01, out_scale=20.0)
    x = to_dev(xb)
    ws = torch.full((sharq.lib().sharq_prep_workspace_bytes(M, K, sharq.NVFP4),), 0xA5, dtype=torch.uint8,
                    device=DEV)
    ob, orr, _ = oracle.prep(xb, n, m, sharq.NVFP4)
    for _ in range(2):
        bb, rr, _ = sharq.prep(x, n, m, sharq.NVFP4, ws=ws)
        torch.cuda.synchronize()
        assert_payload_equal(bb, ob, "backbone")
        assert_payload_equal(rr, orr, "residual")


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
                                   (2000, 4000, 512), (4200, 4100, 256)])
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
    abssum = abs_linear(ob, orr, ow, fmt)
    assert fp32_bound_check(y32, yref, abssum, K) <= 1.0
    assert bf16_bound_check(y16, yref, abssum, K) <= 1.0
    # bf16 rounding alone is up to 2^-8 relative per element, so the Frobenius bound is
    # only meaningful over many outputs; the one-ulp check above covers small cases
    if y16.numel() >= 1024:
        fro = np.linalg.norm(y16.float().cpu().numpy() - yref) / max(np.linalg.norm(yref), 1e-300)
        assert fro <= TOL


@pytest.mark.parametrize("M,N,K", [(600, 512, 8192), (1024, 2048, 4096), (300, 1000, 6144), (40, 300, 4096)])
def test_linear_split_k_matches_oracle(M, N, K):
    """Tiled MXFP4 shapes with few output tiles split K over 2-4 work-groups when the
    workspace holds the partial sums: every output within the fp32 summation bound (any
    summation order), bf16 within one ulp plus it, deterministic across calls; the same
    call with a workspace too small for the partials runs unsplit and meets the same bound.
    A padded, odd ldy takes the reduction's element-wise store."""
    fmt, layout = sharq.MXFP4, sharq.TILED
    need = sharq.lib().sharq_linear_split_workspace_bytes(M, N, K, fmt)
    print(f"[linear split-K] M={M} N={N} K={K} partials={need} B", flush=True)
    assert need > 0, "the shape is meant to split"
    xb, wb = make_shape(M, N, K, seed=M + N + K, dist="laplace", token_sigma=0.3)
    weight = sharq.quantize(to_dev(wb), fmt, layout=layout)
    bb, rr, _ = sharq.prep(to_dev(xb), 2, 4, fmt, layout=layout)
    ws = sharq.workspace(need, DEV)
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    y32 = sharq.linear(bb, rr, weight, sharq.OUT_FP32, ws=ws)
    y32b = sharq.linear(bb, rr, weight, sharq.OUT_FP32, ws=ws)
    y32u = sharq.linear(bb, rr, weight, sharq.OUT_FP32, ws=small)
    y16 = sharq.linear(bb, rr, weight, sharq.OUT_BF16, ws=ws)
    ybuf = torch.zeros((M, N + 3), dtype=torch.bfloat16, device=DEV)
    y16p = sharq.linear(bb, rr, weight, sharq.OUT_BF16, y=ybuf[:, :N], ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), y32b.view(torch.int32)), "split-K is not deterministic"
    assert torch.equal(y16.view(torch.int16), y16p.view(torch.int16)), "padded ldy differs"
    assert torch.all(ybuf[:, N:].view(torch.int16) == 0), "write into the padding"
    ob, orr, _ = oracle.prep(xb, 2, 4, fmt)
    ow = oracle.quantize(wb, fmt)
    yref = oracle.linear(ob, orr, ow, fmt)
    abssum = abs_linear(ob, orr, ow, fmt)
    assert fp32_bound_check(y32, yref, abssum, K) <= 1.0
    assert fp32_bound_check(y32u, yref, abssum, K) <= 1.0
    assert bf16_bound_check(y16, yref, abssum, K) <= 1.0
    assert rel_maxnorm(y32.cpu().numpy().astype(np.float64), yref) <= TOL


def test_linear_split_k_mlp_down_full_size():
    """The MLP block's down projection (M=2048, N=4096, K=14336, MXFP4 2:4, tiled) splits K
    in two: 64 sampled rows against the oracle within the fp32 summation bound."""
    M, N, K = 2048, 4096, 14336
    assert sharq.lib().sharq_linear_split_workspace_bytes(M, N, K, sharq.MXFP4) == 2 * M * N * 4
    print(f"[linear split-K] full size M={M} N={N} K={K}", flush=True)
    xb, wb = make_shape(M, N, K, seed=14, dist="laplace", token_sigma=0.3)
    weight = sharq.quantize(to_dev(wb), sharq.MXFP4, layout=sharq.TILED)
    bb, rr, _ = sharq.prep(to_dev(xb), 2, 4, sharq.MXFP4, layout=sharq.TILED)
    y32 = sharq.linear(bb, rr, weight, sharq.OUT_FP32)  # the binding sizes the workspace for the split
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(M, 64, replace=False))
    ob, orr, _ = oracle.prep(xb[rows], 2, 4, sharq.MXFP4)
    ow = oracle.quantize(wb, sharq.MXFP4)
    yref = oracle.linear(ob, orr, ow, sharq.MXFP4)
    abssum = abs_linear(ob, orr, ow, sharq.MXFP4)
    assert fp32_bound_check(y32.cpu().numpy()[rows].astype(np.float64), yref, abssum, K) <= 1.0


def _random_forward_cases(count=24, seed=20261204):
    """Seeded random configurations of the whole layer: format, layout, pattern, ragged
    M, N and K (a multiple of the format's block), padded rows of X, input distribution
    and output type."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        fmt = int(rng.integers(0, 2))
        layout = sharq.ROWMAJOR if fmt == sharq.NVFP4 else (sharq.TILED if rng.random() < 0.6 else sharq.ROWMAJOR)
        n, m = [(2, 4), (4, 8)][int(rng.integers(0, 2))]
        blk = 16 if fmt == sharq.NVFP4 else 32
        M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 700))]))
        N = int(rng.integers(1, 700))
        K = blk * int(rng.integers(1, 2048 // blk + 1))
        pad = 8 * int(rng.integers(0, 9))
        dist = ["normal", "laplace", "student_t3"][int(rng.integers(0, 3))]
        out = int(rng.integers(0, 2))
        cases.append((i, fmt, layout, n, m, M, N, K, pad, dist, out))
    return cases


@pytest.mark.parametrize("case", _random_forward_cases(), ids=lambda c: f"case{c[0]}")
def test_forward_random_shapes(case):
    """sharq_forward (the launch bench.py times) on seeded random configurations:
    payloads bit for bit, Y within the summation bound of the oracle's exact value."""
    i, fmt, layout, n, m, M, N, K, pad, dist, out = case
    print(f"[forward random] {case}", flush=True)
    xb, wb = make_shape(M, N, K, seed=1000 + i, dist=dist, token_sigma=0.5)
    if pad:
        wide = np.zeros((M, K + pad), np.uint16)
        wide[:, :K] = xb
        x = to_dev(wide)[:, :K]
    else:
        x = to_dev(xb)
    weight = sharq.quantize(to_dev(wb), fmt, layout=layout)
    bufs = (sharq.Payload.empty(M, K, fmt, DEV, layout), sharq.Payload.empty(M, K, fmt, DEV, layout))
    y, (bb, rr) = sharq.forward(x, weight, n, m, out_dtype=out, bufs=bufs)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(xb, n, m, fmt)
    ow = oracle.quantize(wb, fmt)
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")
    assert_payload_equal(weight, ow, "weight")
    yref = oracle.linear(ob, orr, ow, fmt)
    abssum = abs_linear(ob, orr, ow, fmt)
    if out == sharq.OUT_FP32:
        assert rel_maxnorm(y.cpu().numpy().astype(np.float64), yref) <= TOL
        assert fp32_bound_check(y, yref, abssum, K) <= 1.0
    else:
        assert bf16_bound_check(y, yref, abssum, K) <= 1.0


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
    y = y32.cpu().numpy()[rows].astype(np.float64)
    err = rel_maxnorm(y, yref)
    assert err <= TOL, f"{name}: fp32 output max-norm rel err {err}"
    abssum = np.abs(oracle.dequant(oa, w.fmt)[rows]) @ np.abs(oracle.dequant(ow, w.fmt)).T
    assert fp32_bound_check(y, yref, abssum, w.K) <= 1.0


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_linear_workloads_full_compare(name):
    """Full-size shapes in the benchmark's launch configuration (one sharq_forward call),
    every output compared: fp32 max-norm and per-element bound, bf16 per-element bound."""
    w = WORKLOADS[name]
    print(f"[linear] {name} M={w.M} N={w.N} K={w.K} fmt={w.fmt} (all rows)", flush=True)
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
    yref = oracle.linear(ob, orr, ow, w.fmt)
    y = y32.cpu().numpy().astype(np.float64)
    del y32
    err = rel_maxnorm(y, yref)
    assert err <= TOL, f"{name}: fp32 output max-norm rel err {err}"
    abssum = abs_linear(ob, orr, ow, w.fmt)
    worst = fp32_bound_check(y, yref, abssum, w.K)
    assert worst <= 1.0, f"{name}: fp32 output beyond the summation bound ({worst:.3g} of it)"
    del y
    worst = bf16_bound_check(y16, yref, abssum, w.K)
    assert worst <= 1.0, f"{name}: bf16 output beyond one ulp + the summation bound ({worst:.3g} of it)"


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
        y = big[:M * ld].view(M, ld)[:, :N]  # an (M, N) view with row pitch ld
        sharq.linear(bb, rr, weight, sharq.OUT_FP32, y=y)
        torch.cuda.synchronize()
        out = big.cpu().numpy()
        assert np.all(np.isnan(out[M * ld:])), "write past the output"
        assert np.all(np.isnan(out[:M * ld].reshape(M, ld)[:, N:])), "write into the ld padding"
        res.append(out[:M * ld].reshape(M, ld)[:, :N].copy())
    assert np.array_equal(res[0], res[1])


@pytest.mark.parametrize("fmt", [sharq.MXFP4, sharq.NVFP4], ids=["mx", "nv"])
@pytest.mark.parametrize("M,N,K", [(2040, 4090, 128), (1930, 3850, 64), (4400, 4090, 128)])
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


@pytest.mark.parametrize("M,N,K", [(400, 32974, 256), (2048, 8448, 128), (512, 40960, 64)])
def test_linear_tail_of_half_width_tiles(M, N, K):
    """Shapes whose 256 x 256 tiles overflow whole waves of work-groups by at most half a
    wave of whole tile columns (258 tiles: one column of 2; 264: one of 8; 320: 32 of 2)
    run those columns as a second launch of 256 x 128 tiles.  Every output of both paths
    and of the one-operand form is compared with the oracle (fp32 per-element bound, bf16
    one ulp plus the bound), and a padded, odd row pitch gets the same values with nothing
    written into its padding."""
    print(f"[linear] tail columns M={M} N={N} K={K}", flush=True)
    xb, wb = make_shape(M, N, K, seed=17)
    weight = sharq.quantize(to_dev(wb), sharq.MXFP4)
    bb, rr, _ = sharq.prep(to_dev(xb), 2, 4, sharq.MXFP4)
    y32 = sharq.linear(bb, rr, weight, sharq.OUT_FP32)
    y16 = sharq.linear(bb, rr, weight, sharq.OUT_BF16)
    yd = sharq.linear_dense(rr, weight, sharq.OUT_FP32)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(xb, 2, 4, sharq.MXFP4)
    ow = oracle.quantize(wb, sharq.MXFP4)
    yref = oracle.linear(ob, orr, ow)
    abssum = abs_linear(ob, orr, ow, sharq.MXFP4)
    y = y32.cpu().numpy().astype(np.float64)
    assert rel_maxnorm(y, yref) <= TOL
    assert fp32_bound_check(y, yref, abssum, K) <= 1.0, "fp32 output beyond the summation bound"
    assert bf16_bound_check(y16, yref, abssum, K) <= 1.0, "bf16 output beyond one ulp + the bound"
    dref = oracle.linear_dense(orr, ow)
    dabs = np.abs(oracle.dequant(orr, sharq.MXFP4)) @ np.abs(oracle.dequant(ow, sharq.MXFP4)).T
    assert fp32_bound_check(yd.cpu().numpy().astype(np.float64), dref, dabs, K) <= 1.0, "one-operand form"
    ref = y16.view(torch.int16).cpu().numpy()
    ld = N + 3
    big = torch.full(((M + 1) * ld,), -1, dtype=torch.int16, device=DEV)  # 0xFFFF: a bf16 NaN
    yp = big.view(torch.bfloat16)[:M * ld].view(M, ld)[:, :N]
    sharq.linear(bb, rr, weight, sharq.OUT_BF16, y=yp)
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    assert np.all(out[M * ld:] == -1), "write past the output"
    rows = out[:M * ld].reshape(M, ld)
    assert np.all(rows[:, N:] == -1), "write into the row padding"
    assert np.array_equal(rows[:, :N], ref), "values differ from the contiguous output"


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
    with pytest.raises(ValueError, match="layout"):  # the binding's check
        sharq.linear(bb, rr, w_rm)
    # and the library's own, through the C ABI
    y = torch.empty((64, 64), dtype=torch.bfloat16, device=DEV)
    sb, sr, sw = bb.struct(), rr.struct(), w_rm.struct()
    status = sharq.lib().sharq_linear(ctypes.byref(sb), ctypes.byref(sr), 64, ctypes.byref(sw), 64, 128,
                                      sharq.MXFP4, ctypes.c_void_p(y.data_ptr()), 64, sharq.OUT_BF16, None, 0,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == 4  # SHARQ_E_FORMAT


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


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
def test_prep_rmsnorm_every_bf16_value(fmt, layout):
    """Every finite bf16 pattern once, shuffled over 32 rows of K = 2048 (the tiled MXFP4
    form reads each row once): every row's factor is set by near-maximum values, so most
    normalized values land among the subnormals and zeros of either sign."""
    print(f"[prep_rmsnorm] every bf16 value fmt={fmt} layout={layout}", flush=True)
    rng = np.random.default_rng(17)
    xb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xb[(xb & 0x7F80) == 0x7F80] = 0  # infinities and NaN are not part of the contract
    rng.shuffle(xb)
    xb = xb.reshape(32, 2048)
    g = _gain(2048, 3)
    bb, rr, mask = sharq.prep_rmsnorm(to_dev(xb), to_dev(g), 1e-5, 2, 4, fmt, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    yb, _ = oracle.rmsnorm(xb, g, 1e-5)
    ob, orr, omask = oracle.prep(yb, 2, 4, fmt)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("M,K,ldx_pad", [(19, 2048, 0), (33, 2176, 0), (16, 3072, 128), (50, 4096, 0),
                                         (7, 4224, 0), (5, 8192, 0), (6, 8320, 0), (3, 14336, 0),
                                         (9, 16384, 0), (5, 16512, 0), (2, 32768, 0)])
def test_prep_rmsnorm_tiled_row_lengths(n, m, M, K, ldx_pad):
    """Tiled MXFP4 normalized preparation around the one-read kernel's limits: one and
    two steps per wave, wave counts that are not powers of two, a last step past the
    padded row, the longest rows that fit (16384) and longer ones (the two-pass path),
    with ragged row groups; bit for bit."""
    print(f"[prep_rmsnorm] tiled {n}:{m} M={M} K={K} pad={ldx_pad}", flush=True)
    xb, _ = make_shape(M, 8, K, seed=M * 11 + K, dist="normal", token_sigma=0.8)
    g = _gain(K, K + 1)
    if ldx_pad:
        wide = np.zeros((M, K + ldx_pad), np.uint16)
        wide[:, :K] = xb
        x = to_dev(wide)[:, :K]
    else:
        x = to_dev(xb)
    bb, rr, mask = sharq.prep_rmsnorm(x, to_dev(g), 1e-6, n, m, sharq.MXFP4, want_mask=True, layout=sharq.TILED)
    torch.cuda.synchronize()
    yb, _ = oracle.rmsnorm(xb, g, 1e-6)
    ob, orr, omask = oracle.prep(yb, n, m, sharq.MXFP4)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


def test_bf16_rounding_of_the_normalization_is_nearest_even():
    """The packed fp32 -> bf16 conversion the one-read normalized preparation rounds y
    with agrees with round-to-nearest-even on the bits for every finite fp32 pattern."""
    print("[bf16 rounding probe] all 2^32 patterns", flush=True)
    bad, first = sharq.bf16_rounding_probe()
    assert bad == 0, f"{bad} patterns differ, first 0x{first:08x}"


def test_e4m3_block_scale_conversion_follows_the_format():
    """The fp8 conversions the NVFP4 preparation codes and decodes its block scales with
    agree with E4M3's definition (nearest value, ties to the even code, saturating at 448)
    on every fp32 operand with the sign bit clear, and on every code up to 0x7E."""
    print("[e4m3 conversion probe] all 2^31 non-negative patterns, codes 0..0x7E", flush=True)
    bad, first = sharq.e4m3_conversion_probe()
    assert bad == 0, f"{bad} mismatches, first 0x{first:x}"


def _order_sensitive_row(K, big):
    """A row whose fp64 sum of squares depends on the order of the additions: `big` ones
    in the first run of 8, squares of 2^-54 everywhere else (each one lost when added
    alone to a running sum of at least 1, kept when summed among themselves first), and
    a probe in an otherwise zero block 1 whose normalized value, with gain 1.75, sits on
    the bf16 midpoint below a power of two when r is a power of two."""
    x = np.full(K, 2.0 ** -27, np.float32)
    x[:big] = 1.0
    x[32:64] = 0.0
    x[40] = 146 * 2.0 ** -40
    g = np.ones(K, np.float32)
    g[40] = 224 * 2.0 ** -7
    return f32_to_bf16_bits(x), f32_to_bf16_bits(g)


@pytest.mark.parametrize("layout", [sharq.TILED, sharq.ROWMAJOR], ids=["tiled", "rowmajor"])
@pytest.mark.parametrize("K,big,c,n,m", [(2048, 2, 5, 2, 4), (3072, 3, 5, 4, 8), (4096, 1, 6, 2, 4),
                                         (8192, 2, 6, 4, 8), (16384, 4, 6, 2, 4), (32768, 8, 6, 4, 8)])
def test_prep_rmsnorm_follows_the_sum_order(layout, K, big, c, n, m):
    """The normalized preparation reproduces the defined order of the row's sum of squares:
    with S/K = 2^-2c and eps = 2^(-2c-24), a plain left-to-right sum (= big) gives r = 2^c
    and the defined order (slightly more) gives r = 2^c - 2^(c-24), and the probe block's
    scale byte tells the two apart.  Other rows are random."""
    print(f"[prep_rmsnorm] sum order layout={layout} K={K}", flush=True)
    row, g = _order_sensitive_row(K, big)
    eps = 2.0 ** (-2 * c - 24)
    # the construction discriminates: a left-to-right sum lands exactly on `big`
    vals = row.astype(np.uint32) << 16
    left_to_right = 0.0
    for v in vals.view(np.float32).astype(np.float64):
        left_to_right = left_to_right + v * v
    assert left_to_right == big and oracle.row_sumsq(row[None, :])[0] > big
    flat = row.copy()
    flat[(np.arange(K) >= 64) | ((np.arange(K) >= big) & (np.arange(K) < 32))] = 0  # S = big exactly
    y_seq, r_seq = oracle.rmsnorm(flat[None, :], g, eps)
    y_def, r_def = oracle.rmsnorm(row[None, :], g, eps)
    assert r_seq[0] == 2.0 ** c and r_def[0] == np.float32(2.0 ** c - 2.0 ** (c - 24))
    assert oracle.prep(y_seq, n, m)[0].scales[0, 1] != oracle.prep(y_def, n, m)[0].scales[0, 1]

    rnd, _ = make_shape(21, 8, K, seed=K + big, dist="normal")
    xb = np.concatenate([rnd[:9], row[None, :], rnd[9:]])
    bb, rr, mask = sharq.prep_rmsnorm(to_dev(xb), to_dev(g), eps, n, m, sharq.MXFP4, want_mask=True, layout=layout)
    torch.cuda.synchronize()
    yb, _ = oracle.rmsnorm(xb, g, eps)
    ob, orr, omask = oracle.prep(yb, n, m, sharq.MXFP4)
    assert np.array_equal(mask.cpu().numpy(), omask), "mask bits differ"
    assert_payload_equal(bb, ob, "backbone")
    assert_payload_equal(rr, orr, "residual")


@pytest.mark.parametrize("name", ["prefill", "dit"])
def test_prep_rmsnorm_workload_full_size(name):
    """The prefill and DiT workloads' activations through the normalized preparation."""
    w = WORKLOADS[name]
    print(f"[prep_rmsnorm] {name} full size", flush=True)
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


def test_stream_probe_moves_the_bytes():
    """The streaming probe (a measurement aid) reads and writes exactly what it is asked:
    chunk c of the output is chunk c of the input xor c, nothing past write_bytes."""
    print("[stream_probe]", flush=True)
    n_r, n_w = 16 * 5000, 16 * 3001
    src = torch.randint(0, 256, (n_r,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n_w + 4096, dtype=torch.uint8, device=DEV)
    sharq.stream_probe(src, n_r, dst, n_w)
    torch.cuda.synchronize()
    s32 = src.view(torch.int32).cpu().numpy().reshape(-1, 4).astype(np.uint32)
    d32 = dst.view(torch.int32).cpu().numpy().astype(np.uint32)
    want = s32[: n_w // 16].copy()
    want[:, 0] ^= np.arange(n_w // 16, dtype=np.uint32)
    want[:, 1:] ^= np.arange(n_w // 16, dtype=np.uint32)[:, None]
    assert np.array_equal(d32[: n_w // 4].reshape(-1, 4), want)
    assert np.all(d32[n_w // 4:] == 0)


def test_matrix_rate_probe_is_plausible():
    print("[matrix_rate_probe]", flush=True)
    for form in (0, 1):
        cpi, hz = sharq.matrix_rate_probe(form, 20000)
        assert 4 < cpi < 512 and 0.5e9 < hz < 3.5e9, (form, cpi, hz)


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


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS, ids=FL_IDS)
def test_prep_swiglu_every_bf16_gate(fmt, layout):
    """Every finite bf16 pattern as a gate (512 rows x 128: the tiled MXFP4 path looks silu
    up in a table over part of them and applies a rule to the rest), each row's gates in
    shuffled order beside up values in (-1, 1) -- so that h stays finite, as the contract
    asks (|silu(g)| <= |g|)."""
    print(f"[prep_swiglu] every bf16 gate fmt={fmt} layout={layout}", flush=True)
    M, I = 512, 128
    rng = np.random.default_rng(11)
    gates = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    gates[(gates & 0x7F80) == 0x7F80] = 0  # infinities and NaN are not part of the contract
    rng.shuffle(gates)
    gu = np.zeros((M, 2 * I), np.uint16)
    gu[:, :I] = gates.reshape(M, I)
    gu[:, I:] = f32_to_bf16_bits(rng.uniform(-0.99, 0.99, (M, I)).astype(np.float32))
    h = oracle.swiglu(gu, I)
    assert not np.any((h & 0x7F80) == 0x7F80), "the input must keep h finite"
    bb, rr, _ = sharq.prep_swiglu(to_dev(gu), I, 2, 4, fmt, layout=layout)
    torch.cuda.synchronize()
    ob, orr, _ = oracle.prep(h, 2, 4, fmt)
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


# ------------------------------------------------------------------ beyond 32-bit offsets

def _tiled_rows(p, rows):
    """Row-major codes and scales of the given rows of a tiled MXFP4 payload, gathered on
    the device by the layout's definition (codes: fragment (r//32, b//2) at byte
    ((r//32) * Kp/64 + b//2) * 1024, slot (r%32) + 32 (b%2) of 16 bytes; scales: byte b%4
    of word (b//4) * Rp + r), so only the sampled rows travel to the host."""
    Rp, Kp = layout_ref.padded(p.rows, p.K)
    nb = p.K // 32
    r = torch.as_tensor(rows, dtype=torch.int64, device=p.codes.device)[:, None]
    b = torch.arange(nb, dtype=torch.int64, device=p.codes.device)[None, :]
    slot = ((r // 32) * (Kp // 64) + b // 2) * 1024 + ((r % 32) + 32 * (b % 2)) * 16
    idx = (slot[:, :, None] + torch.arange(16, device=p.codes.device)).reshape(-1)
    codes = p.codes[idx].reshape(len(rows), p.K // 2).cpu().numpy()
    sidx = ((b // 4) * Rp + r) * 4 + b % 4
    scales = p.scales[sidx.reshape(-1)].reshape(len(rows), nb).cpu().numpy()
    return codes, scales


def test_prep_and_linear_beyond_32bit_offsets():
    """X of 2.2 M x 2048 bf16 (4.5 G elements, 9 GB): more row groups than one launch's
    grid holds, code payloads past 2^31 bytes and X past 2^31 elements, so every 64-bit
    offset of the preparation (tiled and row-major) and of the tiled GEMM is exercised.
    X repeats a seeded 4096-row block, each repetition scaled by a power of two (exact in
    bf16), so the oracle computes the sampled rows from the block alone (MXFP4 rows are
    independent); the rows sampled sit at the launch and 2^31 boundaries and at the ends."""
    M, K, N, base_rows = 2_200_000, 2048, 256, 4096
    print(f"[big] prep + linear M={M} K={K} N={N} (sampled rows)", flush=True)
    xb_base, wb = make_shape(base_rows, N, K, seed=2024, out_frac=0.01, out_scale=30.0)
    shift = lambda i: (i // base_rows) % 7 - 3  # the power of two applied to row i
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    base = to_dev(xb_base)
    for j in range((M + base_rows - 1) // base_rows):  # exact: power-of-two factors
        n = min(base_rows, M - j * base_rows)
        x[j * base_rows:j * base_rows + n] = base[:n] * (2.0 ** shift(j * base_rows))
    del base
    weight = sharq.quantize(to_dev(wb), sharq.MXFP4)

    launch_rows = 65535 * 16
    rows = sorted({0, 1, 31, 32, launch_rows - 1, launch_rows, launch_rows + 1, 2 * launch_rows,
                   (1 << 31) // K - 1, (1 << 31) // K, (1 << 31) // (K // 2) - 1, (1 << 31) // (K // 2),
                   (1 << 31) // (K // 2) + 33, M - 33, M - 32, M - 2, M - 1}
                  | set(int(v) for v in np.random.default_rng(7).integers(0, M, 15)))
    xs = np.stack([f32_to_bf16_bits(bf16_bits_to_f32(xb_base[i % base_rows]) * np.float32(2.0 ** shift(i)))
                   for i in rows])
    ob, orr, _ = oracle.prep(xs, 2, 4, sharq.MXFP4)
    ow = oracle.quantize(wb, sharq.MXFP4)

    bb, rr, _ = sharq.prep(x, 2, 4, sharq.MXFP4, layout=sharq.TILED)
    torch.cuda.synchronize()
    for p, want, what in ((bb, ob, "backbone"), (rr, orr, "residual")):
        c, s = _tiled_rows(p, rows)
        bad = np.nonzero((c != want.codes).any(axis=1) | (s != want.scales).any(axis=1))[0]
        assert bad.size == 0, f"tiled {what}: rows {[rows[i] for i in bad[:8]]} differ"

    y = sharq.linear(bb, rr, weight, out_dtype=sharq.OUT_FP32)
    torch.cuda.synchronize()
    ys = y[torch.as_tensor(rows, device=DEV)].cpu().numpy().astype(np.float64)
    del y, bb, rr
    yref = oracle.linear(ob, orr, ow)
    assert rel_maxnorm(ys, yref) <= TOL
    worst = fp32_bound_check(ys, yref, abs_linear(ob, orr, ow, sharq.MXFP4), K)
    assert worst <= 1.0, f"sampled GEMM rows beyond the summation bound ({worst:.3g} of it)"

    bb, rr, _ = sharq.prep(x, 2, 4, sharq.MXFP4, layout=sharq.ROWMAJOR)
    torch.cuda.synchronize()
    del x
    ridx = torch.as_tensor(rows, device=DEV)
    for p, want, what in ((bb, ob, "backbone"), (rr, orr, "residual")):
        c = p.codes.view(M, K // 2)[ridx].cpu().numpy()
        s = p.scales.view(M, K // 32)[ridx].cpu().numpy()
        assert np.array_equal(c, want.codes) and np.array_equal(s, want.scales), f"row-major {what} differs"
    # the row-major GEMM over the same (row-major) payloads
    y = sharq.linear(bb, rr, weight.convert(sharq.ROWMAJOR), out_dtype=sharq.OUT_FP32)
    torch.cuda.synchronize()
    ys = y[ridx].cpu().numpy().astype(np.float64)
    del y
    worst = fp32_bound_check(ys, yref, abs_linear(ob, orr, ow, sharq.MXFP4), K)
    assert worst <= 1.0, f"row-major GEMM rows beyond the summation bound ({worst:.3g} of it)"


@pytest.mark.parametrize("K", [1024, 1040])
def test_linear_nvfp4_payloads_past_2gib(K):
    """NVFP4 GEMM with activation payloads past 2 GiB (rows x K/2 >= 2^31 bytes): the
    kernels taken there (streaming for K % 64 == 0, register-staged otherwise) against the
    oracle on sampled rows.  The payloads are seeded synthetic FP4 data (random codes, E4M3
    block scales around 1, tensor scales that are not powers of two) repeating a 4096-row
    block, so the oracle sees only the block's rows; none comes from the library."""
    M, N, base_rows = ((1 << 31) // (K // 2)) + 4100, 128, 4096
    print(f"[big] nvfp4 linear M={M} N={N} K={K} (sampled rows)", flush=True)
    rng = np.random.default_rng(99 + K)

    def synth(rows, tscale):
        codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
        scales = rng.integers(0x28, 0x49, (rows, K // 16), dtype=np.uint8)
        return oracle.Payload(codes, scales, np.float32(tscale))

    ob, orr, ow = synth(base_rows, 0.7), synth(base_rows, 0.03125 * 1.3), synth(N, 0.011)

    def dev_payload(p, rows):
        reps = (rows + base_rows - 1) // base_rows
        codes = torch.from_numpy(p.codes).to(DEV).repeat(reps, 1)[:rows].contiguous().view(-1)
        scales = torch.from_numpy(p.scales).to(DEV).repeat(reps, 1)[:rows].contiguous().view(-1)
        ts = torch.full((4,), float(p.tscale), dtype=torch.float32, device=DEV)
        return sharq.Payload(codes, scales, ts, sharq.NVFP4, sharq.ROWMAJOR, rows, K)

    bb, rr, w = dev_payload(ob, M), dev_payload(orr, M), dev_payload(ow, N)
    y = sharq.linear(bb, rr, w, out_dtype=sharq.OUT_FP32)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 127, 128, (1 << 31) // (K // 2) - 1, (1 << 31) // (K // 2), M - 129, M - 1}
                  | set(int(v) for v in np.random.default_rng(5).integers(0, M, 8)))
    ys = y[torch.as_tensor(rows, device=DEV)].cpu().numpy().astype(np.float64)
    del y, bb, rr
    pick = [i % base_rows for i in rows]
    sb = oracle.Payload(ob.codes[pick], ob.scales[pick], ob.tscale)
    sr = oracle.Payload(orr.codes[pick], orr.scales[pick], orr.tscale)
    yref = oracle.linear(sb, sr, ow, sharq.NVFP4)
    assert rel_maxnorm(ys, yref) <= TOL
    worst = fp32_bound_check(ys, yref, abs_linear(sb, sr, ow, sharq.NVFP4), K)
    assert worst <= 1.0, f"sampled rows beyond the summation bound ({worst:.3g} of it)"


def test_prep_nvfp4_beyond_32bit_elements():
    """NVFP4 preparation of X with more than 2^31 elements (1.1 M x 2048 bf16).  X repeats
    one seeded 4096-row block unchanged, so both tensor maxima -- of X and of the residual
    -- are the block's, and the oracle's preparation of the block alone fixes every row's
    payload and both tensor scales; rows sampled at the 2^31-element boundary, the ends
    and at random are compared bit for bit."""
    M, K, base_rows = 1_100_000, 2048, 4096
    print(f"[big] nvfp4 prep M={M} K={K} (sampled rows)", flush=True)
    xb_base, _ = make_shape(base_rows, 16, K, seed=404, dist="laplace", out_frac=0.01, out_scale=20.0)
    reps = (M + base_rows - 1) // base_rows
    x = to_dev(xb_base).repeat(reps, 1)[:M].contiguous()
    bb, rr, _ = sharq.prep(x, 2, 4, sharq.NVFP4)
    torch.cuda.synchronize()
    del x
    ob, orr, _ = oracle.prep(xb_base, 2, 4, sharq.NVFP4)
    rows = sorted({0, 1, (1 << 31) // K - 1, (1 << 31) // K, (1 << 31) // K + 1, M - 2, M - 1}
                  | set(int(v) for v in np.random.default_rng(3).integers(0, M, 12)))
    ridx = torch.as_tensor(rows, device=DEV)
    pick = [i % base_rows for i in rows]
    for p, want, what in ((bb, ob, "backbone"), (rr, orr, "residual")):
        c = p.codes.view(M, K // 2)[ridx].cpu().numpy()
        s = p.scales.view(M, K // 16)[ridx].cpu().numpy()
        assert np.array_equal(c, want.codes[pick]), f"{what} codes differ"
        assert np.array_equal(s, want.scales[pick]), f"{what} scales differ"
        assert np.float32(p.tensor_scale[0].item()) == np.float32(want.tscale), f"{what} tensor scale differs"
