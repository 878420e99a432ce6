"""Seeded random inputs.

Every stream comes from numpy's PCG64 seeded by SeedSequence(base, spawn_key=
path), so any (layer, sequence, purpose) block can be regenerated on its own,
in any order, on the CPU or before an upload to the GPU.
"""

from __future__ import annotations

import numpy as np


def rng_for(base: int, *path: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(base, spawn_key=tuple(path))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns uint16 bits.

    Used only to produce bf16 inputs from normal samples (inputs contain no NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, outlier_frac: float = 0.0,
                outlier_mult: float = 20.0) -> np.ndarray:
    """N(0,1) samples as bf16 bits; a Bernoulli(outlier_frac) subset is scaled by outlier_mult."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)
