"""Seeded synthetic inputs shaped like Flux-12B linear layers.

This module only draws random numbers and casts them to bf16: it holds none of
the quantizer's or the GEMM's arithmetic, so the CPU oracle and the HIP path
can both be fed from it.

Recipe: ``numpy.random.Generator(PCG64(seed))``; ``standard_normal`` in float64
scaled to the stated standard deviation, cast to float32, then to bf16 with
round-to-nearest-even (torch's CPU cast).  Tensors are drawn in the order the
workload lists them.  Returned arrays are bf16 *bit patterns* (uint16).

Workloads (rows x cols of each bf16 tensor; the hidden size 3072, QKV width
9216 and MLP width 12288 are Flux-12B's, token counts are per-GPU microbatch
shapes):
  tiny   seed 0: A 256x512 N(0,1), W 384x512 N(0,1)
  dual   seed 1: X 4600x3072 N(0,1); entries with uniform draw < 1e-3 scaled
                 by 100 (outliers); one aligned 32x32 all-zero tile per 1024
                 rows (rows [1024g, 1024g+32), cols [64g, 64g+32))
  qkv    seed 2: A 4608x3072 N(0,1), W 9216x3072 N(0,0.02)
  fc1    seed 3: X 9216x3072 N(0,1), W 12288x3072 N(0,0.02), dY 9216x12288 N(0,1e-3)
  fc2    seed 4: X 18432x12288 GELU(N(0,1)) (exact erf form),
                 W 3072x12288 N(0,0.02), dY 18432x3072 N(0,1e-3)
"""
from __future__ import annotations

import numpy as np

try:  # torch is the bf16 caster (RNE); it is present wherever this package runs
    import torch
except Exception:  # pragma: no cover
    torch = None


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std) as bf16 bits."""
    return bf16_bits((rng.standard_normal(shape, dtype=np.float64) * std).astype(np.float32))


def gelu_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """GELU (exact erf form) of N(0,1), as bf16 bits."""
    z = torch.from_numpy(rng.standard_normal(shape, dtype=np.float64))
    g = torch.nn.functional.gelu(z, approximate="none")
    return bf16_bits(g.to(torch.float32).numpy())


def tiny(seed: int = 0):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = normal(rng, (256, 512), 1.0)
    w = normal(rng, (384, 512), 1.0)
    return {"A": a, "W": w}


def dual(seed: int = 1, rows: int = 4600, cols: int = 3072):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float64)
    mask = rng.random((rows, cols)) < 1e-3
    x[mask] *= 100.0
    for g in range(rows // 1024 + (1 if rows % 1024 else 0)):
        r0, c0 = 1024 * g, 64 * g
        if r0 < rows and c0 < cols:
            x[r0:r0 + 32, c0:c0 + 32] = 0.0
    return {"X": bf16_bits(x.astype(np.float32))}


def qkv(seed: int = 2):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = normal(rng, (4608, 3072), 1.0)
    w = normal(rng, (9216, 3072), 0.02)
    return {"A": a, "W": w}


def fc1(seed: int = 3):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = normal(rng, (9216, 3072), 1.0)
    w = normal(rng, (12288, 3072), 0.02)
    dy = normal(rng, (9216, 12288), 1e-3)
    return {"X": x, "W": w, "dY": dy}


def fc2(seed: int = 4, tokens: int = 18432):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = gelu_normal(rng, (tokens, 12288))
    w = normal(rng, (3072, 12288), 0.02)
    dy = normal(rng, (tokens, 3072), 1e-3)
    return {"X": x, "W": w, "dY": dy}


def random_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, std) bf16 tensor for parity sweeps."""
    return normal(np.random.Generator(np.random.PCG64(seed)), shape, std)
