"""Seeded synthetic inputs for the attention backward (random numbers and bf16 rounding only).

This module holds no attention arithmetic. It draws Q, K, V and dO from a fixed
PCG64 stream and rounds them to bf16, so that the GPU path, the CPU oracle and the
benchmark all receive the same bytes.

Workload shape (DASH paper, section 4.1 "Benchmark Settings"): bf16 random inputs,
16 384 tokens in total, hidden size 2048, head dim 64 or 128. Values are standard
normal, matching the paper's "BF16 precision random inputs".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "make_qkvdo",
    "config_seed",
]


def bf16_round_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen raw bf16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def config_seed(index: int) -> int:
    """Seed of workload number `index` (0 = tiny, 1..4 = the large configs)."""
    return 1000 + int(index)


def make_qkvdo(B: int, H: int, Hkv: int, N: int, d: int, seed: int) -> dict:
    """Draw Q, K, V, dO ~ N(0, 1) in that order from PCG64(seed); return bf16 bit arrays.

    Shapes: q, do -> [B, H, N, d]; k, v -> [B, Hkv, N, d] (uint16 bf16 bits, C order).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv), ("do", H)):
        x = rng.standard_normal((B, heads, N, d), dtype=np.float32)
        out[name] = bf16_round_bits(x)
    return out
