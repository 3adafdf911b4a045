"""Seeded synthetic inputs for the SharQ linear layer.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws random numbers and casts them to bf16 bit patterns; it holds none of the
method's arithmetic (no mask, no scale, no FP4 rounding) and imports nothing
from the rest of the package or from the oracle.

The workloads stand in for the pages' LLM-serving and video-DiT linear layers
(SharQ, arXiv 2606.26587: abstract, Figure 3 and Figure 4), whose layer shapes
the pages do not print.  The shapes, distributions and outlier structure are the
five configurations below.  Weights are random (no checkpoints), drawn as bf16
and quantized by whichever side consumes them.

Draw order for every workload, from ``numpy.random.default_rng(seed)``:
  1. base X [M, K] in float64 from the named distribution;
  2. outlier channels ``rng.choice(K, n_out, replace=False)``, multiplied by the factor;
  3. optionally a per-token scale ``rng.lognormal(0, sigma, M)`` (column vector);
  4. W [N, K] ~ Normal(0, 0.02) in float64;
  5. both cast float64 -> float32 -> bf16 with round-to-nearest-even.
"""
from dataclasses import dataclass, field

import numpy as np

MXFP4 = 0
NVFP4 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    n: int
    m: int
    fmt: int
    dist: str
    out_frac: float = 0.0
    out_count: int = 0
    out_scale: float = 1.0
    token_sigma: float = 0.0
    w_std: float = 0.02
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def n_out(self) -> int:
        if self.out_count:
            return self.out_count
        return int(round(self.out_frac * self.K))

    def flops_effective(self) -> float:
        return 2.0 * self.M * self.N * self.K


WORKLOADS = {
    "tiny": Workload("tiny", 16, 512, 512, 2, 4, MXFP4, "normal", out_count=4, out_scale=20.0,
                     note="X[16,512] N(0,1), 4 outlier channels x20; W[512,512]; 2:4; MXFP4"),
    "decode": Workload("decode", 16, 14336, 4096, 2, 4, MXFP4, "student_t3", out_frac=0.01,
                       out_scale=30.0,
                       note="X[16,4096] Student-t(3), 1% outlier channels x30; W[14336,4096]; 2:4; MXFP4"),
    "prefill": Workload("prefill", 4096, 4096, 4096, 2, 4, MXFP4, "normal", out_frac=0.005,
                        out_scale=50.0, token_sigma=0.5,
                        note="X[4096,4096] N(0,1), 0.5% outlier channels x50, per-token LogNormal(0,0.5); "
                             "W[4096,4096]; 2:4; MXFP4"),
    "mlp_down_nvfp4": Workload("mlp_down_nvfp4", 2048, 4096, 14336, 2, 4, NVFP4, "laplace",
                               out_frac=0.01, out_scale=20.0,
                               note="X[2048,14336] Laplace(0,1), 1% outlier channels x20; W[4096,14336]; "
                                    "2:4; NVFP4"),
    "dit": Workload("dit", 32760, 3072, 3072, 4, 8, MXFP4, "normal", out_frac=0.02, out_scale=15.0,
                    note="X[32760,3072] N(0,1), 2% outlier channels x15; W[3072,3072]; 4:8; MXFP4"),
}


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _base(rng, dist, shape):
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "student_t3":
        return rng.standard_t(3.0, shape)
    if dist == "laplace":
        return rng.laplace(0.0, 1.0, shape)
    raise ValueError(f"unknown distribution {dist}")


def make_activation(rng, M, K, dist="normal", n_out=0, out_scale=1.0, token_sigma=0.0):
    """Draw X [M,K] with outlier channels and an optional per-token scale, as bf16 bits."""
    x = _base(rng, dist, (M, K))
    if n_out:
        ch = rng.choice(K, n_out, replace=False)
        x[:, ch] *= out_scale
    if token_sigma:
        x *= rng.lognormal(0.0, token_sigma, M)[:, None]
    return f32_to_bf16_bits(x.astype(np.float32))


def make_inputs(w: Workload, with_weight=True, rows=None):
    """Return (x_bits [M,K], w_bits [N,K] or None) for a workload.

    ``rows`` truncates M after drawing (the draws are those of the full workload,
    so a row sample is the same bytes as the full input's first rows).
    """
    rng = np.random.default_rng(w.seed)
    x = make_activation(rng, w.M, w.K, w.dist, w.n_out, w.out_scale, w.token_sigma)
    wb = None
    if with_weight:
        wb = f32_to_bf16_bits(rng.normal(0.0, w.w_std, (w.N, w.K)).astype(np.float32))
    if rows is not None:
        x = x[:rows].copy()
    return x, wb


def make_shape(M, N, K, seed, dist="normal", out_frac=0.01, out_scale=20.0, token_sigma=0.0):
    """Inputs for an arbitrary shape with the same recipe (used by shape sweeps)."""
    rng = np.random.default_rng(seed)
    n_out = int(round(out_frac * K))
    x = make_activation(rng, M, K, dist, n_out, out_scale, token_sigma)
    wb = f32_to_bf16_bits(rng.normal(0.0, 0.02, (N, K)).astype(np.float32))
    return x, wb


def adversarial_activation(M, K, seed=0):
    """Rows built to hit the corner cases of the codec: ties within groups, all-zero
    groups and blocks, +0/-0, bf16 subnormals, huge and tiny blocks, and values on
    the E2M1 rounding midpoints and in the saturation band relative to a power-of-two
    block maximum.  Returned as bf16 bits [M, K] (K a multiple of 32)."""
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    x = np.zeros((M, K), np.float32)
    # magnitudes as multiples of a quarter on a grid that includes every E2M1
    # midpoint (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) and the band above 6.
    grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 7.5],
                    np.float32)
    for i in range(M):
        kind = i % 8
        for b in range(K // 32):
            e = int(rng.integers(-20, 20))
            if kind == 0:    # exact grid / midpoint values, block max 4*2^e
                blk = rng.choice(grid[:13], 32) * np.float32(2.0 ** e)
                blk[rng.integers(0, 32)] = np.float32(4 * 2.0 ** e)
            elif kind == 1:  # saturation band: block max in (6, 8) * 2^e
                blk = rng.choice(grid, 32) * np.float32(2.0 ** e)
                blk[rng.integers(0, 32)] = np.float32(7.5 * 2.0 ** e)
            elif kind == 2:  # heavy ties: few distinct magnitudes
                blk = rng.choice(np.array([0, 1, 1, 2], np.float32), 32) * np.float32(2.0 ** e)
            elif kind == 3:  # all-zero blocks with signed zeros
                blk = np.where(rng.random(32) < 0.5, np.float32(0.0), np.float32(-0.0))
            elif kind == 4:  # bf16 subnormals and tiny normals
                bits = rng.integers(1, 0x00FF, 32).astype(np.uint32) << 16
                blk = bits.view(np.float32).copy()
            elif kind == 5:  # huge blocks near the bf16 maximum
                blk = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** 120)
            elif kind == 6:  # one outlier and otherwise tiny values
                blk = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** -12)
                blk[rng.integers(0, 32)] = np.float32(3.0e4)
            else:            # ordinary normal values
                blk = rng.standard_normal(32).astype(np.float32)
            sign = np.where(rng.random(32) < 0.5, np.float32(-1), np.float32(1))
            x[i, b * 32:(b + 1) * 32] = blk * sign
    return f32_to_bf16_bits(x)


@dataclass(frozen=True)
class MlpBlock:
    """A Llama-3.1-8B-shaped MLP block (hidden H, intermediate I) over M tokens:
    gate/up projection (one linear over the concatenated [gate; up] weights, N = 2I),
    SwiGLU, down projection (K = I), each projection a SharQ layer."""
    name: str
    M: int
    H: int
    I: int
    n: int
    m: int
    fmt: int
    dist: str = "normal"
    out_frac: float = 0.01
    out_scale: float = 20.0
    w_std: float = 0.02
    seed: int = 0
    note: str = field(default="", compare=False)

    def flops_effective(self) -> float:
        return 2.0 * self.M * self.H * (2 * self.I) + 2.0 * self.M * self.I * self.H


MLP_BLOCKS = {
    "mlp_block": MlpBlock("mlp_block", 2048, 4096, 14336, 2, 4, MXFP4,
                          note="X[2048,4096] N(0,1), 1% outlier channels x20; W_gate_up[28672,4096], "
                               "W_down[4096,14336] N(0,0.02); SwiGLU; 2:4; MXFP4"),
    "mlp_block_small": MlpBlock("mlp_block_small", 64, 512, 1024, 2, 4, MXFP4,
                                note="the same recipe at a size the oracle finishes in seconds"),
}


def make_mlp_inputs(b: MlpBlock):
    """Draw order: X [M,H] (distribution, outlier channels), then W_gate_up [2I,H], then
    W_down [H,I], all from numpy.random.default_rng(seed); returns bf16 bits."""
    rng = np.random.default_rng(b.seed)
    x = make_activation(rng, b.M, b.H, b.dist, int(round(b.out_frac * b.H)), b.out_scale)
    wgu = f32_to_bf16_bits(rng.normal(0.0, b.w_std, (2 * b.I, b.H)).astype(np.float32))
    wd = f32_to_bf16_bits(rng.normal(0.0, b.w_std, (b.H, b.I)).astype(np.float32))
    return x, wgu, wd
