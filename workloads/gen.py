"""Seeded input generation.

Every tensor is drawn in fp64 from ``numpy.random.default_rng(seed)`` in the
order the workload lists, then rounded once, round-to-nearest-even, to its
storage dtype.  bf16 tensors are returned as ``uint16`` bit patterns, fp32
tensors as ``float32``.  Nothing here depends on the method being computed.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .spec import TensorSpec, WorkloadSpec

_F32_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_STEP = 2.0 ** -133


def bf16_bits_from_f64(x) -> np.ndarray:
    """Round fp64 values to bf16 (round-to-nearest-even, one rounding).

    Normal range: drop the low 45 of fp64's 52 mantissa bits with RNE, after
    which the value is exactly representable in fp32 and its top 16 bits are
    the bf16 pattern.  Below fp32's normal range bf16 is subnormal with a
    fixed step of 2^-133, rounded with numpy's half-to-even ``round``.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)
    rounded = (bits + half_minus_one + lsb) & ~np.uint64((1 << 45) - 1)
    y = rounded.view(np.float64)
    tiny = np.abs(x) < _F32_MIN_NORMAL
    if np.any(tiny):
        y = np.where(tiny, np.round(x / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP, y)
    y32 = y.astype(np.float32)
    return (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of a stored tensor."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def draw_tensor(rng: np.random.Generator, t: TensorSpec) -> np.ndarray:
    z = rng.standard_normal(t.shape)          # fp64
    std = float(np.sqrt(t.var))
    if t.dist == "normal":
        v = z * std
    elif t.dist == "abs_normal":
        v = np.abs(z * std)
    elif t.dist == "one_plus_normal":
        v = 1.0 + z * std
    elif t.dist == "row_shift_normal":
        # N(0, var) plus one N(0, 1) offset per row (drawn after the values):
        # rows whose means are of the order of their spread
        v = z * std + rng.standard_normal((t.shape[0], 1))
    else:
        raise ValueError(t.dist)
    if t.dtype == "bf16":
        return bf16_bits_from_f64(v)
    if t.dtype == "f32":
        return v.astype(np.float32)
    raise ValueError(t.dtype)


def make_inputs(spec: WorkloadSpec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every tensor of ``spec`` in its listed order from one generator."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    return {t.name: draw_tensor(rng, t) for t in spec.tensors}
