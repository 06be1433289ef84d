"""Seeded synthetic inputs for the LM-head path (shared by tests, the oracle
checks and the benchmark).

This module only draws random numbers; it holds none of the method's
arithmetic.  Conversion of FP32 draws to BF16 storage goes through torch's
own CPU cast (round to nearest, ties to even), a library routine that is
neither the oracle nor the HIP path.

Every draw uses ``numpy.random.default_rng(seed)`` with a fresh generator per
workload, in the order documented on each function.  "p% of rows" means the
exact count round(p * n) chosen by ``rng.choice(n, k, replace=False)``.

Workloads (shapes from the pages' benchmark and exactness sweeps):

* ``tiny_exact``  x [16 x 512], W [1024 x 512] integers uniform in [-8, 8],
  targets uniform in [0, 1024), no ignored rows (the integer exactness
  construction of Megatron-LM "Add mixed-precision (FP32) LM output logits",
  sections "Tests" and "Method", seed 1234).
* ``lmhead_128``  M=128, K=4096, V=32768; x ~ N(0,1), W ~ N(0, 0.02^2);
  5% of rows ignored (-100).
* ``lmhead_1024`` M=1024, K=8192, V=32768; x ~ N(0,1), W ~ N(0, 0.02^2).
* ``xent_131k``   logits FP32 [8192 x 131072] ~ N(0, 3^2), 1% of rows get +30
  at a random column, 2% of rows ignored.
* ``step_4096``   M=4096, K=16384, V=131072; x ~ N(0,1), W ~ N(0, 0.01^2).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED = 1234
IGNORE_INDEX = -100

# Rows drawn per chunk for large normal arrays (bounds host memory).
_CHUNK_ELEMS = 1 << 26


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 storage bits via torch's CPU cast (nearest, ties to even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def int_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Small integers (|v| <= 256) are exact in BF16."""
    a = np.asarray(a)
    if a.size and np.abs(a).max() > 256:
        raise ValueError("integer too large to be exact in BF16")
    return f32_to_bf16_bits(a.astype(np.float32))


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) drawn as float32 in row chunks, stored as BF16 bits."""
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        chunk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            chunk *= np.float32(sigma)
        out[r0:r1] = f32_to_bf16_bits(chunk)
    return out


def normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    rows, cols = shape
    out = np.empty(shape, dtype=np.float32)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            out[r0:r1] *= np.float32(sigma)
    return out


def pick_rows(rng: np.random.Generator, n: int, frac: float) -> np.ndarray:
    k = int(round(frac * n))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(n, k, replace=False)).astype(np.int64)


@dataclass
class GemmInputs:
    x: np.ndarray            # uint16 BF16 bits [M, K]
    W: np.ndarray            # uint16 BF16 bits [V, K]
    target: np.ndarray       # int32 [M]
    ignore_index: int = IGNORE_INDEX
    meta: dict = field(default_factory=dict)


@dataclass
class XentInputs:
    logits: np.ndarray       # float32 [n, V]
    target: np.ndarray       # int32 [n]
    ignore_index: int = IGNORE_INDEX
    spike_rows: Optional[np.ndarray] = None
    spike_cols: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)


def integer_gemm(M: int, K: int, V: int, seed: int = SEED, lo: int = -8, hi: int = 8,
                 with_targets: bool = True) -> GemmInputs:
    """Integer operands uniform in [lo, hi] (inclusive).  Draw order: x, W,
    then targets uniform in [0, V)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, (M, K))
    W = rng.integers(lo, hi + 1, (V, K))
    t = rng.integers(0, V, M).astype(np.int32) if with_targets else np.zeros(M, np.int32)
    return GemmInputs(int_to_bf16_bits(x), int_to_bf16_bits(W), t,
                      meta={"kind": "integer", "range": (lo, hi), "seed": seed})


def integer_operands(shapes, seed: int = SEED, lo: int = -8, hi: int = 8):
    """BF16 bit arrays of integers uniform in [lo, hi], drawn in the order of
    `shapes` from one generator."""
    rng = np.random.default_rng(seed)
    return [int_to_bf16_bits(rng.integers(lo, hi + 1, tuple(s))) for s in shapes]


def random_shapes(n: int, seed: int, m_set, v_set, k8_max: int):
    """n random problem shapes for parity sweeps, one generator, drawn in this
    order per case: M from m_set, K = 8 * U[1, k8_max), V from v_set, then the
    extra leading-dimension padding of x, W (multiples of 8 elements, 0 - 16),
    of a BF16 [M, V] operand (0 or 8) and of an FP32 [M, V] operand (0 or 4)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice(m_set))
        K = int(8 * rng.integers(1, k8_max))
        V = int(rng.choice(v_set))
        out.append({"M": M, "K": K, "V": V,
                    "pad_x": int(8 * rng.integers(0, 3)), "pad_w": int(8 * rng.integers(0, 3)),
                    "pad_g": int(8 * rng.integers(0, 2)), "pad_z": int(4 * rng.integers(0, 2))})
    return out


def uniform_targets(n: int, V: int, ignore_frac: float, seed: int) -> np.ndarray:
    """Targets uniform in [0, V), then round(ignore_frac * n) rows set to the
    ignore index (chosen without replacement)."""
    rng = np.random.default_rng(seed)
    t = rng.integers(0, V, n).astype(np.int32)
    k = int(round(ignore_frac * n))
    if k:
        t[rng.choice(n, k, replace=False)] = IGNORE_INDEX
    return t


def tiny_exact(seed: int = SEED) -> GemmInputs:
    """x [16 x 512], W [1024 x 512] integers in [-8, 8], targets in [0, 1024)."""
    g = integer_gemm(16, 512, 1024, seed)
    g.meta.update(name="tiny_exact", dloss=1.0 / 16)
    return g


def normal_gemm(M: int, K: int, V: int, sigma_w: float, seed: int = SEED,
                ignore_frac: float = 0.0) -> GemmInputs:
    """Draw order: x ~ N(0,1) [M, K], W ~ N(0, sigma_w^2) [V, K], targets
    uniform in [0, V), then the ignored rows."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    W = normal_bf16(rng, (V, K), sigma_w)
    t = rng.integers(0, V, M).astype(np.int32)
    ign = pick_rows(rng, M, ignore_frac)
    t[ign] = IGNORE_INDEX
    return GemmInputs(x, W, t, meta={"kind": "normal", "sigma_w": sigma_w, "seed": seed,
                                     "ignored_rows": ign})


def lmhead_128(seed: int = SEED) -> GemmInputs:
    g = normal_gemm(128, 4096, 32768, 0.02, seed, ignore_frac=0.05)
    g.meta["name"] = "lmhead_128"
    return g


def lmhead_1024(seed: int = SEED) -> GemmInputs:
    g = normal_gemm(1024, 8192, 32768, 0.02, seed)
    g.meta["name"] = "lmhead_1024"
    return g


def step_4096(seed: int = SEED) -> GemmInputs:
    g = normal_gemm(4096, 16384, 131072, 0.01, seed)
    g.meta["name"] = "step_4096"
    return g


def xent_logits(n: int, V: int, sigma: float = 3.0, spike_frac: float = 0.01,
                spike: float = 30.0, ignore_frac: float = 0.02,
                seed: int = SEED) -> XentInputs:
    """Draw order: logits ~ N(0, sigma^2) [n, V]; spike rows; their columns
    uniform in [0, V); targets uniform in [0, V); ignored rows (independent of
    the spikes).  Spike rows get +spike added at their column."""
    rng = np.random.default_rng(seed)
    z = normal_f32(rng, (n, V), sigma)
    srows = pick_rows(rng, n, spike_frac)
    scols = rng.integers(0, V, srows.size).astype(np.int64)
    z[srows, scols] += np.float32(spike)
    t = rng.integers(0, V, n).astype(np.int32)
    ign = pick_rows(rng, n, ignore_frac)
    t[ign] = IGNORE_INDEX
    return XentInputs(z, t, IGNORE_INDEX, srows, scols,
                      meta={"sigma": sigma, "spike": spike, "seed": seed, "ignored_rows": ign})


def xent_131k(seed: int = SEED, n: int = 8192) -> XentInputs:
    x = xent_logits(n, 131072, seed=seed)
    x.meta["name"] = "xent_131k"
    return x


# The pages' GEMM timing grid: M in {16, 128, 1024} x K in {1024 ... 16384}
# (powers of two) x N = 32,768 (Megatron-LM "Add mixed-precision (FP32) LM
# output logits", section "Tests", the benchmark bullet).
GEMM_GRID_M = (16, 128, 1024)
GEMM_GRID_K = (1024, 2048, 4096, 8192, 16384)
GEMM_GRID_V = 32768

# The integer exactness sweep widths (same page, section "Method").
INT_SWEEP_K = (512, 1024, 2048, 4096, 8192, 16384)
