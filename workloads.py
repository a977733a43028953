"""Seeded synthetic inputs for the FP8 quantization / GEMM workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the quantization or GEMM arithmetic.  Both the CPU oracle
and the HIP library consume the same host buffers made here.

Generator: numpy ``default_rng(seed)`` (PCG64), draws in float64, scaled in
float64, then rounded to float32 (``astype``) and, for bf16 workloads, on to
bf16 (round to nearest even, via torch's CPU cast).  bf16 arrays are returned as numpy
``uint16`` bit patterns.

Workloads (all sizes overridable so the same recipe serves small parity cases):
  tensor_fp32   1024x1024 fp32, N(0,1)*300, 16 entries set to +-2000 (seed 0)
  delayed_step  8192x8192 bf16, N(0, sigma_t), sigma_t = 0.01*1.05^t, with
                0.1% of the entries (chosen without replacement) replaced by
                N(0, 50*sigma_t) draws (seed 1000+t)
  block_weight  7168x4096 bf16, N(0, 0.02) (seed 1)
  block_act     4096x7168 bf16, N(0,1) with 1% of the columns (chosen without
                replacement) replaced by standard Student-t(3) draws (seed 2)
  gemm_pair     two 8192x8192 bf16 N(0,1) operands (seeds 3, 4)
  mlp_block     X 4096x4096 N(0,1) (seed 5), W 14336x4096 N(0,0.02) (seed 6),
                dY 4096x14336 N(0,1e-3) (seed 7), all bf16
The second parameter of N(.,.) is a standard deviation.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """Round float64 draws to float32, then to bf16 (nearest even, torch's CPU
    cast), and return the bf16 bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for host-side checks)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def tensor_fp32(rows: int = 1024, cols: int = 1024, seed: int = 0, n_outliers: int = 16,
                outlier: float = 2000.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * 300.0
    n = rows * cols
    k = min(n_outliers, n)
    idx = rng.choice(n, k, replace=False)
    sgn = rng.choice(np.array([-1.0, 1.0]), k)
    flat = x.reshape(-1)
    flat[idx] = outlier * sgn
    return x.astype(np.float32)


def delayed_sigma(t: int) -> float:
    return 0.01 * (1.05 ** t)


def delayed_step(t: int, rows: int = 8192, cols: int = 8192, outlier_frac: float = 0.001,
                 seed_base: int = 1000) -> np.ndarray:
    rng = np.random.default_rng(seed_base + t)
    sigma = delayed_sigma(t)
    n = rows * cols
    x = rng.standard_normal(n) * sigma
    k = int(round(outlier_frac * n))
    if k:
        idx = rng.choice(n, k, replace=False)
        x[idx] = rng.standard_normal(k) * (50.0 * sigma)
    return to_bf16_bits(x.reshape(rows, cols))


def block_weight(rows: int = 7168, cols: int = 4096, seed: int = 1, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((rows, cols)) * std)


def block_act(rows: int = 4096, cols: int = 7168, seed: int = 2, heavy_frac: float = 0.01) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    k = int(round(heavy_frac * cols))
    if k:
        c = rng.choice(cols, k, replace=False)
        x[:, c] = rng.standard_t(3, (rows, k))
    return to_bf16_bits(x)


def gemm_pair(m: int = 8192, n: int = 8192, k: int = 8192, seeds=(3, 4)):
    a = np.random.default_rng(seeds[0]).standard_normal((m, k))
    b = np.random.default_rng(seeds[1]).standard_normal((n, k))
    return to_bf16_bits(a), to_bf16_bits(b)


def mlp_block(tokens: int = 4096, hidden: int = 4096, ffn: int = 14336, seeds=(5, 6, 7)):
    x = np.random.default_rng(seeds[0]).standard_normal((tokens, hidden))
    w = np.random.default_rng(seeds[1]).standard_normal((ffn, hidden)) * 0.02
    dy = np.random.default_rng(seeds[2]).standard_normal((tokens, ffn)) * 1e-3
    return to_bf16_bits(x), to_bf16_bits(w), to_bf16_bits(dy)


def special_values_f32() -> np.ndarray:
    """A short list of float32 edge values: signed zeros, infinities, NaNs of
    both signs, the extremes of the binary32 range and subnormals."""
    bits = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000,
                     0x7F800001, 0x7FFFFFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x80000001,
                     0x007FFFFF, 0x00800000, 0x3F800000, 0xBF800000], dtype=np.uint32)
    return bits.view(np.float32)


def parallel_map(fn, items, workers: int = 8):
    """Generate several seeded inputs at once (numpy's generators release the
    GIL while filling large arrays); results keep the order of ``items``."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
