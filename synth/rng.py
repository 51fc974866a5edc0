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

import os

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


def _normal_pairs(seed: int, tag: int, p0: int, p1: int) -> np.ndarray:
    """Normals 2*p0 .. 2*p1-1 of a stream: Box-Muller on uniform pairs p0 .. p1-1."""
    z = splitmix64(seed, tag, 2 * (p1 - p0), offset=2 * p0)
    u = (z >> np.uint64(11)).astype(np.float64)
    u *= 1.0 / 9007199254740992.0
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))  # log(1 - u1): u1 < 1 so the log is finite
    t = (2.0 * np.pi) * u2
    out = np.empty(2 * (p1 - p0), dtype=np.float64)
    np.multiply(r, np.cos(t), out=out[0::2])
    np.multiply(r, np.sin(t), out=out[1::2])
    return out


_CHUNK_PAIRS = 1 << 20


def _chunks(m: int):
    return [(p, min(m, p + _CHUNK_PAIRS)) for p in range(0, m, _CHUNK_PAIRS)]


def _pool_map(fn, items):
    """Map over chunks with threads (numpy releases the GIL); order-preserving
    and independent of the thread count, since each chunk is a pure function of
    its stream offsets."""
    if len(items) <= 1:
        return [fn(i) for i in items]
    from concurrent.futures import ThreadPoolExecutor

    workers = min(len(items), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """n standard normals (fp64) by Box-Muller over consecutive uniform pairs."""
    m = (n + 1) // 2
    out = np.empty(2 * m, dtype=np.float64)

    def work(c):
        p0, p1 = c
        out[2 * p0:2 * p1] = _normal_pairs(seed, tag, p0, p1)

    _pool_map(work, _chunks(m))
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
    """A tensor of N(mean, std^2) values in ``dtype`` ("f32" -> float32, "bf16" -> uint16 bits).

    Each value is mean + std * z in fp64, rounded RNE to fp32 (then RNE to bf16).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    n = int(np.prod(shape))
    m = (n + 1) // 2
    out = np.empty(2 * m, dtype=np.float32 if dtype == "f32" else np.uint16)

    def work(c):
        p0, p1 = c
        x = (mean + std * _normal_pairs(seed, tag, p0, p1)).astype(np.float32)
        out[2 * p0:2 * p1] = x if dtype == "f32" else f32_to_bf16_bits(x)

    _pool_map(work, _chunks(m))
    return out[:n].reshape(shape)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of the values a device sees for ``x`` stored as ``dtype``."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
