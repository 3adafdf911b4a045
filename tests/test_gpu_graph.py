"""Steps captured into HIP graphs (as `bench.py --graph` issues them) replay the same
results as the eager launches, and eager repeats reproduce their own results exactly.

A step is the preparation + the fused linear (or the MLP block's four calls) on fixed
buffers.  The eager step runs first; the graph is captured on torch's capture stream,
then replayed several times with eager work and synchronizations between the replays
(outputs overwritten with a sentinel, an unrelated matrix product), and every replay's
payloads and output are compared with the eager ones byte for byte: the kernels are
deterministic, so a replay must reproduce them exactly.
"""
import numpy as np
import pytest
import torch

from activation_sparsity_fp4_sharq_amd import sharq
from activation_sparsity_fp4_sharq_amd.workloads import make_shape

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 4


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def snapshot(tensors):
    return [t.detach().clone() for t in tensors]


def spoil(tensors):
    for t in tensors:
        t.view(torch.uint8).fill_(0xA5)


def check_replays(step, outputs):
    step()
    torch.cuda.synchronize()
    want = snapshot(outputs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    junk = torch.randn(256, 256, device=DEV)
    for rep in range(REPLAYS):
        spoil(outputs)
        junk = (junk @ junk) / 256.0  # eager work on the same stream between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outputs, want)):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"replay {rep}: output {i} differs"


def check_repeats(step, outputs):
    """Eager repeats of the same step reproduce their outputs exactly (no races)."""
    step()
    torch.cuda.synchronize()
    want = snapshot(outputs)
    for rep in range(REPLAYS):
        spoil(outputs)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outputs, want)):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"eager repeat {rep}: output {i} differs"


def payload_tensors(p):
    # the preparation writes an NVFP4 payload's tensor scale (the first of the 4 floats the
    # binding allocates); an MXFP4 payload has none
    return [p.codes, p.scales] + ([p.tensor_scale[:1]] if p.fmt == sharq.NVFP4 else [])


CASES = [
    (16, 512, 512, sharq.MXFP4, 4, sharq.TILED),       # small-M kernel
    (300, 384, 640, sharq.MXFP4, 8, sharq.TILED),      # tiled LDS-DMA kernel, ragged M and N
    (200, 160, 384, sharq.MXFP4, 4, sharq.ROWMAJOR),  # row-major kernel
    (130, 256, 512, sharq.NVFP4, 4, None),             # NVFP4: three preparation passes + reductions
    (600, 512, 8192, sharq.MXFP4, 4, sharq.TILED),     # 6 tiles: K split in four + the ordered reduction
    (400, 32974, 128, sharq.MXFP4, 8, sharq.TILED),    # 258 tiles: 256 + a tail of 128-column tiles
]


def make_step(M, N, K, fmt, m, layout):
    xb, wb = make_shape(M, N, K, seed=M + N + K)
    x = to_dev(xb)
    w = sharq.quantize(to_dev(wb), fmt, layout=layout)
    kw = {} if layout is None else {"layout": layout}
    bb = sharq.Payload.empty(M, K, fmt, DEV, **kw)
    rr = sharq.Payload.empty(M, K, fmt, DEV, **kw)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = sharq.workspace(max(sharq.lib().sharq_prep_workspace_bytes(M, K, fmt),
                             sharq.lib().sharq_linear_workspace_bytes(M, N, K, fmt),
                             sharq.lib().sharq_linear_split_workspace_bytes(M, N, K, fmt)), DEV)

    def step():
        sharq.prep(x, m // 2, m, fmt, out=(bb, rr), ws=ws)
        sharq.linear(bb, rr, w, sharq.OUT_BF16, y=y, ws=ws)

    return step, payload_tensors(bb) + payload_tensors(rr) + [y]


@pytest.mark.parametrize("M,N,K,fmt,m,layout", CASES)
def test_step_eager_repeats_identical(M, N, K, fmt, m, layout):
    print(f"[repeat] M={M} N={N} K={K} fmt={fmt} m={m} layout={layout}", flush=True)
    check_repeats(*make_step(M, N, K, fmt, m, layout))


@pytest.mark.parametrize("M,N,K,fmt,m,layout", CASES)
def test_step_graph_replays_match_eager(M, N, K, fmt, m, layout):
    print(f"[graph] M={M} N={N} K={K} fmt={fmt} m={m} layout={layout}", flush=True)
    check_replays(*make_step(M, N, K, fmt, m, layout))


def test_mlp_block_graph_replays_match_eager():
    from activation_sparsity_fp4_sharq_amd.workloads import MLP_BLOCKS, make_mlp_inputs
    b = MLP_BLOCKS["mlp_block_small"]
    print(f"[graph] mlp block M={b.M} H={b.H} I={b.I}", flush=True)
    xb, wgub, wdb = make_mlp_inputs(b)
    x = to_dev(xb)
    wgu = sharq.quantize(to_dev(wgub), b.fmt)
    wd = sharq.quantize(to_dev(wdb), b.fmt)
    b1, r1 = sharq.Payload.empty(b.M, b.H, b.fmt, DEV), sharq.Payload.empty(b.M, b.H, b.fmt, DEV)
    b2, r2 = sharq.Payload.empty(b.M, b.I, b.fmt, DEV), sharq.Payload.empty(b.M, b.I, b.fmt, DEV)
    gu = torch.empty((b.M, 2 * b.I), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((b.M, b.H), dtype=torch.bfloat16, device=DEV)
    ws = sharq.workspace(max(sharq.lib().sharq_prep_workspace_bytes(b.M, max(b.H, b.I), b.fmt),
                             sharq.lib().sharq_linear_workspace_bytes(b.M, 2 * b.I, max(b.H, b.I), b.fmt)), DEV)

    def step():
        sharq.prep(x, b.n, b.m, b.fmt, out=(b1, r1), ws=ws)
        sharq.linear(b1, r1, wgu, sharq.OUT_BF16, y=gu, ws=ws)
        sharq.prep_swiglu(gu, b.I, b.n, b.m, b.fmt, out=(b2, r2), ws=ws)
        sharq.linear(b2, r2, wd, sharq.OUT_BF16, y=y, ws=ws)

    check_replays(step, payload_tensors(b1) + payload_tensors(r1) + [gu] + payload_tensors(b2)
                  + payload_tensors(r2) + [y])


@pytest.mark.parametrize("M,N,K,fmt", [(16, 512, 512, sharq.MXFP4), (300, 384, 640, sharq.MXFP4),
                                       (130, 256, 512, sharq.NVFP4)])
def test_bind_forward_matches_forward(M, N, K, fmt):
    """The pre-marshalled sharq_forward call gives the same payloads and output as
    `forward`, on every invocation."""
    print(f"[bind] M={M} N={N} K={K} fmt={fmt}", flush=True)
    xb, wb = make_shape(M, N, K, seed=3 * M + K)
    x = to_dev(xb)
    w = sharq.quantize(to_dev(wb), fmt)
    y_ref, (b_ref, r_ref) = sharq.forward(x, w)
    torch.cuda.synchronize()
    want = snapshot(payload_tensors(b_ref) + payload_tensors(r_ref) + [y_ref])
    call = sharq.bind_forward(x, w)
    y, (bb, rr) = call.outputs
    outs = payload_tensors(bb) + payload_tensors(rr) + [y]
    for rep in range(3):
        spoil(outs)
        call()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"call {rep}: output {i} differs"


def test_two_streams_concurrently_match_sequential():
    """Two steps on two streams at once (different inputs, their own buffers and
    workspaces) give the same bytes as each step alone: the library keeps no state
    between calls beyond per-device kernel attributes."""
    print("[streams] two concurrent steps", flush=True)
    cases = [(300, 512, 640, sharq.MXFP4), (130, 256, 512, sharq.NVFP4)]
    runs = []
    for M, N, K, fmt in cases:
        xb, wb = make_shape(M, N, K, seed=M * 7 + K)
        x = to_dev(xb)
        w = sharq.quantize(to_dev(wb), fmt)
        y, (bb, rr) = sharq.forward(x, w, n=2, m=4)
        torch.cuda.synchronize()
        want = snapshot(payload_tensors(bb) + payload_tensors(rr) + [y])
        runs.append((x, w, bb, rr, y, want))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for x, w, bb, rr, y, want in runs:
            spoil(payload_tensors(bb) + payload_tensors(rr) + [y])
        torch.cuda.synchronize()
        for (x, w, bb, rr, y, want), s in zip(runs, streams):
            with torch.cuda.stream(s):
                sharq.forward(x, w, n=2, m=4, bufs=(bb, rr), y=y)
        torch.cuda.synchronize()
        for i, (x, w, bb, rr, y, want) in enumerate(runs):
            outs = payload_tensors(bb) + payload_tensors(rr) + [y]
            for j, (got, ref) in enumerate(zip(outs, want)):
                assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"rep {rep}: case {i} output {j}"
