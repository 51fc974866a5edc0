"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds random-number plumbing only: no step of the attention head
(positions, angles, normalisation, rotation, softmax) is computed here.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser constants are Vigna's
published ones).  Each tensor draws from its own stream whose initial state is
``seed XOR tag``; the n-th output (n = 0, 1, ...) is the finaliser applied to
``state + (n + 1) * GOLDEN``, which is exactly what the sequential generator
returns, so the stream can be produced vectorised.

Uniforms take the top 53 bits.  Normals use Box-Muller on consecutive pairs.
Values are rounded round-to-nearest-even to fp32 and, for bf16 tensors, again
RNE from fp32 to bf16; bf16 tensors are held as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream tags, one per drawn tensor.
TAG_Q, TAG_K, TAG_V, TAG_GAMMA_Q, TAG_GAMMA_K, TAG_LENS = 1, 2, 3, 4, 5, 6


def splitmix64(seed: int, tag: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs ``offset .. offset+n-1`` of the SplitMix64 stream seeded ``seed ^ tag``."""
    state = np.uint64((seed ^ tag) & 0xFFFFFFFFFFFFFFFF)
    idx = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = state + idx * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform(seed: int, tag: int, n: int) -> np.ndarray:
    """n uniforms in [0, 1) from the top 53 bits of each output (fp64)."""
    z = splitmix64(seed, tag, n)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """n standard normals (fp64) by Box-Muller over consecutive uniform pairs."""
    m = (n + 1) // 2
    u = uniform(seed, tag, 2 * m)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))  # log(1 - u1): u1 < 1 so the log is finite
    t = (2.0 * np.pi) * u2
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns.

    NaN stays a quiet NaN; finite values round to the nearest bf16 (ties to even).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    nan = np.isnan(x)
    rounded = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_tensor(seed: int, tag: int, shape, dtype: str, mean: float = 0.0, std: float = 1.0):
    """A tensor of N(mean, std^2) values in ``dtype`` ("f32" -> float32, "bf16" -> uint16 bits)."""
    n = int(np.prod(shape))
    x = (mean + std * normal(seed, tag, n)).astype(np.float32).reshape(shape)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of the values a device sees for ``x`` stored as ``dtype``."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
