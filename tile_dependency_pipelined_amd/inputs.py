"""Seeded synthetic inputs for the GEMM-chain workloads.

This module holds no arithmetic of the method: it only draws matrices with
numpy's PCG64 generator and stores them in the element type of the chain.
Both the HIP path's tests/benchmark and the CPU oracle consume what it makes.

Recipe: fp64 standard normals from ``numpy.random.default_rng(seed)``, scaled
by the stated standard deviation, cast to float32, and for bf16 chains
rounded to nearest-even bf16 bit patterns.  Seeds: X uses ``1000*cfg``, the
weight of layer l (1-based) uses ``1000*cfg + l``.  A variance written
N(0, 1/fan_in) means standard deviation 1/sqrt(fan_in).

The workload shapes follow the paper's evaluation shape scaled to one GPU:
X of "sequence length" rows times square 8192 weights, BF16 in/out with FP32
accumulation (CTA-Pipelining, §III-C and §IV-A).
"""
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

F32 = 0
BF16 = 1
ACT_NONE = 0
ACT_GELU_TANH = 1


@dataclass(frozen=True)
class ChainConfig:
    key: str
    cfg_id: int
    description: str
    dtype: int
    M: int
    widths: Tuple[int, ...]
    acts: Tuple[int, ...]
    x_std: float
    w_stds: Tuple[float, ...]
    tile: Optional[Tuple[int, int]] = None  # fixed by the workload, else chosen

    @property
    def n_layers(self) -> int:
        return len(self.widths) - 1

    @property
    def flops(self) -> float:
        return float(sum(2 * self.M * self.widths[l] * self.widths[l + 1]
                         for l in range(self.n_layers)))

    def min_bytes(self) -> int:
        """X + every W + Y, each touched once (the algorithmic byte count)."""
        es = 4 if self.dtype == F32 else 2
        n = self.M * self.widths[0] + self.M * self.widths[-1]
        n += sum(self.widths[l] * self.widths[l + 1] for l in range(self.n_layers))
        return n * es


def _s(fan):
    return 1.0 / math.sqrt(fan)


CONFIGS = {
    "c1": ChainConfig("c1", 1, "2-layer GEMM fp32, X 128x512, W 512x512 x2, 64x64 tiles",
                      F32, 128, (512, 512, 512), (ACT_NONE, ACT_NONE), 1.0,
                      (_s(512), _s(512)), tile=(64, 64)),
    "c2": ChainConfig("c2", 2, "2-layer GEMM bf16, X 512x4096, W 4096x4096 x2",
                      BF16, 512, (4096, 4096, 4096), (ACT_NONE, ACT_NONE), 1.0,
                      (1 / 64.0, 1 / 64.0)),
    "c3": ChainConfig("c3", 3, "2-layer GEMM bf16, X 2048x8192, W 8192x8192 x2",
                      BF16, 2048, (8192, 8192, 8192), (ACT_NONE, ACT_NONE), 1.0,
                      (_s(8192), _s(8192))),
    "c4": ChainConfig("c4", 4, "4-layer GEMM chain bf16, X 1024x8192, W 8192x8192 x4",
                      BF16, 1024, (8192,) * 5, (ACT_NONE,) * 4, 1.0, (_s(8192),) * 4),
    "c5": ChainConfig("c5", 5, "MLP up/down bf16, X 256x8192, W1 8192x28672 + tanh-GeLU, "
                      "W2 28672x8192", BF16, 256, (8192, 28672, 8192),
                      (ACT_GELU_TANH, ACT_NONE), 1.0, (_s(8192), _s(28672))),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_matrix(shape, std: float, seed: int, dtype: int) -> np.ndarray:
    """A seeded N(0, std^2) matrix in the chain's element type."""
    rng = np.random.default_rng(seed)
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16 if dtype == BF16 else np.float32)
    step = max(1, (1 << 24) // max(cols, 1))  # bound the fp64 scratch
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        block = (rng.standard_normal((r1 - r0, cols)) * std).astype(np.float32)
        out[r0:r1] = f32_to_bf16_bits(block) if dtype == BF16 else block
    return out


def chain_inputs(M: int, widths, dtype: int, x_std: float, w_stds, cfg_id: int,
                 rows: Optional[Tuple[int, int]] = None):
    """X (M x K0) and the list of W_l, seeded as described in the module doc.
    ``rows`` = (r0, r1) draws X fully but returns only those rows."""
    X = normal_matrix((M, widths[0]), x_std, 1000 * cfg_id, dtype)
    Ws: List[np.ndarray] = [
        normal_matrix((widths[l], widths[l + 1]), w_stds[l], 1000 * cfg_id + l + 1, dtype)
        for l in range(len(widths) - 1)]
    if rows is not None:
        X = np.ascontiguousarray(X[rows[0]:rows[1]])
    return X, Ws


def config_inputs(cfg: ChainConfig):
    return chain_inputs(cfg.M, cfg.widths, cfg.dtype, cfg.x_std, cfg.w_stds, cfg.cfg_id)


def signed_permutation(n: int, seed: int, dtype: int, scale_pow2: int = 0) -> np.ndarray:
    """A random signed permutation matrix scaled by 2**scale_pow2 (exact in
    every element type).  Used for bit-exact plumbing checks."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    signs = rng.choice(np.array([-1.0, 1.0]), size=n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = signs * (2.0 ** scale_pow2)
    return f32_to_bf16_bits(P) if dtype == BF16 else P


def small_int_matrix(shape, seed: int, dtype: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Seeded small integers (exact in bf16 and fp32)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(a) if dtype == BF16 else a
