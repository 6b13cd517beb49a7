"""Seeded synthetic inputs for the fp16 NT GEMM workloads.

This module only draws numbers: it holds none of the GEMM's arithmetic and
is shared, unchanged, by the oracle-side tests and the GPU-side tests and
benchmark.  Every array is IEEE binary16 (numpy ``float16``) in the layouts
the GEMM takes: A row-major M x K, B row-major N x K.

Shapes follow the pages' workloads: the 128 x 128 x 64 single output tile
and the multi-tile / K-loop steps of page "构建 Tiled GEMM" ("Building a
Tiled GEMM", mlc.ai, sections "第 1 步" .. "第 3 步"), and the 8192^3 fp16
problem that page "如何用 Croqtile 一步步优化矩阵乘法内核" measures
throughout (header and section "性能一览").  The ragged 3000 x 5000 x 2050
shape and the skinny 64 x 16384 x 8192 linear-layer shape extend those
with tails and an HBM-bound case.  The pages fix no value distribution
(page 2's harness draws ``torch.randn``); the distributions below are stated
per workload.

Draws use numpy's PCG64 (``default_rng(seed)``) in float64 and are rounded to
fp16 by numpy's ``astype`` (round to nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    a_dist: str          # "uniform" | "normal_scaled" | "normal_0.02"
    b_dist: str
    seeds: tuple         # (seed_A, seed_B) for the random variant
    int_seeds: tuple     # (seed_A, seed_B) for the integer {-2..2} variant
    sample_seed: int | None = None   # seed of the sampled-entry check, if any


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tile_128x128x64", 128, 128, 64, "uniform", "uniform",
                 (1001, 1002), (1011, 1012)),
        Workload("square_1024", 1024, 1024, 1024, "uniform", "uniform",
                 (2001, 2002), (2011, 2012)),
        Workload("ragged_3000x5000x2050", 3000, 5000, 2050, "normal_scaled", "normal_scaled",
                 (3001, 3002), (3011, 3012)),
        Workload("skinny_64x16384x8192", 64, 16384, 8192, "uniform", "normal_0.02",
                 (4001, 4002), (4011, 4012)),
        Workload("square_8192", 8192, 8192, 8192, "uniform", "uniform",
                 (5001, 5002), (5011, 5012), sample_seed=5003),
        # few output tiles, long K: the stream-K form's case
        Workload("deep_1024x1024x16384", 1024, 1024, 16384, "uniform", "uniform",
                 (6001, 6002), (6011, 6012)),
        # one GPU's share when 8192^3 and the skinny shape are split over
        # B's rows (N) on eight GPUs
        Workload("shard_8192x1024x8192", 8192, 1024, 8192, "uniform", "uniform",
                 (7001, 7002), (7011, 7012), sample_seed=7003),
        Workload("shard_64x2048x8192", 64, 2048, 8192, "uniform", "normal_0.02",
                 (8001, 8002), (8011, 8012)),
    )
}

HEADLINE = "square_8192"


def _draw(rng: np.random.Generator, dist: str, rows: int, K: int) -> np.ndarray:
    shape = (rows, K)
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal_scaled":
        x = rng.standard_normal(size=shape) / np.sqrt(K)
    elif dist == "normal_0.02":
        x = 0.02 * rng.standard_normal(size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float16)


def random_inputs(w: Workload, M: int | None = None, N: int | None = None,
                  K: int | None = None):
    """The random variant of workload ``w`` (optionally at another shape)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    A = _draw(np.random.default_rng(w.seeds[0]), w.a_dist, M, K)
    B = _draw(np.random.default_rng(w.seeds[1]), w.b_dist, N, K)
    return A, B


def integer_inputs(w: Workload, M: int | None = None, N: int | None = None,
                   K: int | None = None):
    """Integer-valued entries, uniform over {-2, -1, 0, 1, 2}."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    A = np.random.default_rng(w.int_seeds[0]).integers(-2, 3, size=(M, K), dtype=np.int8)
    B = np.random.default_rng(w.int_seeds[1]).integers(-2, 3, size=(N, K), dtype=np.int8)
    return A.astype(np.float16), B.astype(np.float16)


def uniform_inputs(seed: int, M: int, N: int, K: int, lo: float = -1.0, hi: float = 1.0):
    """Free-shape uniform[lo, hi] inputs (edge-case sweeps)."""
    rng = np.random.default_rng(seed)
    A = rng.uniform(lo, hi, size=(M, K)).astype(np.float16)
    B = rng.uniform(lo, hi, size=(N, K)).astype(np.float16)
    return A, B


def integer_free(seed: int, M: int, N: int, K: int, lo: int = -2, hi: int = 2):
    """Free-shape integer inputs uniform over {lo..hi}."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, size=(M, K), dtype=np.int16).astype(np.float16)
    B = rng.integers(lo, hi + 1, size=(N, K), dtype=np.int16).astype(np.float16)
    return A, B


def coarse_uniform(seed: int, M: int, N: int, K: int, step: float = 2.0 ** -6,
                   lim: float = 2.0):
    """Free-shape inputs uniform over the multiples of ``step`` in
    [-lim, lim] (both exact in fp16).  With the defaults every product is a
    multiple of 2^-12 below 4 in magnitude, so any sum of 64 of them has at
    most 20 significant bits and is exact in fp32, whatever the order."""
    rng = np.random.default_rng(seed)
    n = int(round(lim / step))
    A = (rng.integers(-n, n + 1, size=(M, K)) * step).astype(np.float16)
    B = (rng.integers(-n, n + 1, size=(N, K)) * step).astype(np.float16)
    return A, B


def random_bits(seed: int, shape, finite_max: float | None = None) -> np.ndarray:
    """Uniformly random fp16 bit patterns over all finite values (subnormals,
    zeros and +-65504 included); optionally restricted to |x| <= finite_max."""
    rng = np.random.default_rng(seed)
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    filled = 0
    while filled < out.size:
        cand = rng.integers(0, 65536, size=2 * (out.size - filled) + 16, dtype=np.uint32)
        cand = cand.astype(np.uint16)
        v = cand.view(np.float16)
        ok = np.isfinite(v)
        if finite_max is not None:
            ok &= np.abs(v.astype(np.float64)) <= finite_max
        cand = cand[ok][: out.size - filled]
        out[filled: filled + cand.size] = cand
        filled += cand.size
    return out.reshape(shape).view(np.float16)


def sample_indices(w: Workload, count: int = 4096):
    """``count`` distinct (row, col) positions of D drawn without replacement
    from the workload's sample seed."""
    seed = w.sample_seed if w.sample_seed is not None else w.seeds[0] + 2
    flat = np.random.default_rng(seed).choice(w.M * w.N, size=count, replace=False)
    return (flat // w.N).astype(np.int64), (flat % w.N).astype(np.int64)


def edge_lines(extent: int, tile: int) -> np.ndarray:
    """Rows (or columns) of D at tile edges: the first, second, last and
    first-of-next of the first two tiles and of the last full tile, the last
    two of the extent, and the fixed probes 63/64/127/128/255/256."""
    full = (extent // tile) * tile
    cand = {0, 1, tile - 1, tile, 2 * tile - 1, 2 * tile, full - 1, full,
            extent - 2, extent - 1, 63, 64, 127, 128, 255, 256}
    return np.array(sorted(c for c in cand if 0 <= c < extent), dtype=np.int64)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float values -> bfloat16 bit patterns (uint16): round the fp32 value to
    its upper 16 bits, nearest with ties to even (input preparation only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_uniform(seed: int, M: int, N: int, K: int):
    """bfloat16 A [M, K], B [N, K], uniform[-1, 1] (bit patterns, uint16)."""
    rng = np.random.default_rng(seed)
    return (to_bf16_bits(rng.uniform(-1.0, 1.0, size=(M, K))),
            to_bf16_bits(rng.uniform(-1.0, 1.0, size=(N, K))))


def bf16_integers(seed: int, M: int, N: int, K: int, lo: int = -2, hi: int = 2):
    """bfloat16 A, B with integer entries in {lo..hi} (exact in bfloat16)."""
    rng = np.random.default_rng(seed)
    return (to_bf16_bits(rng.integers(lo, hi + 1, size=(M, K))),
            to_bf16_bits(rng.integers(lo, hi + 1, size=(N, K))))


# FP8 inputs.  Format codes as in the C ABI: 0 = E4M3, 1 = E5M2.
FP8_MAX = {0: 448.0, 1: 57344.0}


def fp8_quantize(x: np.ndarray, fmt: int):
    """Per-tensor FP8 quantisation (input preparation only): the scale maps
    the largest magnitude to the format's largest finite value, and x / scale
    is rounded to the nearest FP8 value by torch's float8 cast.  Returns the
    FP8 bytes (uint8) and the fp32 dequantisation scale."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = np.float32(amax / FP8_MAX[fmt]) if amax > 0 else np.float32(1.0)
    dt = torch.float8_e5m2 if fmt else torch.float8_e4m3fn
    q = torch.from_numpy(x / scale).to(dt).view(torch.uint8).numpy().copy()
    return q, scale


def fp8_normal(seed: int, M: int, N: int, K: int, fa: int = 0, fb: int = 0):
    """FP8 A [M, K] and B [N, K] quantised from standard normal values, each
    with its own per-tensor scale; returns (A, B, scale) with scale the fp32
    product of the two dequantisation scales."""
    rng = np.random.default_rng(seed)
    A, sa = fp8_quantize(rng.standard_normal((M, K), dtype=np.float32), fa)
    B, sb = fp8_quantize(rng.standard_normal((N, K), dtype=np.float32), fb)
    return A, B, float(np.float32(sa * sb))


def fp8_channelwise(seed: int, M: int, N: int, K: int, fa: int = 0, fb: int = 0):
    """Inputs of the per-channel FP8 product (input preparation only), after
    the GEMM-optimisation article at www.lqnn.cn, section 4.2: A (activations,
    standard normal) quantised with one per-tensor scale, B (weights,
    N(0, 0.02^2) with per-row magnitudes spread over [0.25, 4] so that the
    channel scales differ) with one scale per row mapping that row's largest
    magnitude to the format's largest finite value.  Returns (A, B, a_scale,
    b_scale) with b_scale N fp32 values."""
    import torch
    rng = np.random.default_rng(seed)
    A, sa = fp8_quantize(rng.standard_normal((M, K), dtype=np.float32), fa)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
         * rng.uniform(0.25, 4.0, (N, 1)).astype(np.float32))
    amax = np.abs(W).max(axis=1) if K else np.zeros(N, np.float32)
    sb = np.where(amax > 0, amax / np.float32(FP8_MAX[fb]), 1.0).astype(np.float32)
    dt = torch.float8_e5m2 if fb else torch.float8_e4m3fn
    B = torch.from_numpy(np.ascontiguousarray(W / sb[:, None])).to(dt).view(torch.uint8).numpy().copy()
    return A, B, float(sa), sb


def fp8_integers(seed: int, M: int, N: int, K: int, fa: int = 0, fb: int = 0, lo: int = -4,
                 hi: int = 4):
    """FP8 A, B with integer entries in {lo..hi} (exact in both formats for
    |v| <= 4)."""
    import torch
    rng = np.random.default_rng(seed)
    out = []
    for rows, fmt in ((M, fa), (N, fb)):
        v = rng.integers(lo, hi + 1, size=(rows, K)).astype(np.float32)
        dt = torch.float8_e5m2 if fmt else torch.float8_e4m3fn
        out.append(torch.from_numpy(v).to(dt).view(torch.uint8).numpy().copy())
    return out[0], out[1]
