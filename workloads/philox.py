"""Philox-4x32-10 counter-based generator (host side, numpy).

The generator is the one published by Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11): a 4x32-bit counter and a 2x32-bit
key go through ten rounds of two 32x32->64-bit multiplies with the published
multipliers, xors with the key, and a Weyl-sequence key bump between rounds.

Counter convention used by the synthetic workloads: counter = (index_lo,
index_hi, tensor_tag, sub), key = (seed_lo, seed_hi).  Each counter yields four
uint32 words.  This module holds no arithmetic of the eviction method.
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox-4x32 rounds on uint32 arrays; returns four uint32 arrays."""
    c0 = np.asarray(c0, np.uint32).astype(np.uint64)
    c1 = np.asarray(c1, np.uint32).astype(np.uint64)
    c2 = np.asarray(c2, np.uint32).astype(np.uint64)
    c3 = np.asarray(c3, np.uint32).astype(np.uint64)
    k0 = np.uint32(k0)
    k1 = np.uint32(k1)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = np.uint32((int(k0) + int(_W0)) & 0xFFFFFFFF)
        k1 = np.uint32((int(k1) + int(_W1)) & 0xFFFFFFFF)
    return (c0.astype(np.uint32), c1.astype(np.uint32), c2.astype(np.uint32),
            c3.astype(np.uint32))


def words(seed: int, tag: int, index: np.ndarray, sub: int = 0):
    """Four uint32 words per 64-bit index for (seed, tag, sub)."""
    index = np.asarray(index, np.uint64)
    lo = (index & _MASK).astype(np.uint32)
    hi = (index >> np.uint64(32)).astype(np.uint32)
    n = lo.shape
    return philox4x32_10(lo, hi, np.full(n, tag & 0xFFFFFFFF, np.uint32),
                         np.full(n, sub & 0xFFFFFFFF, np.uint32),
                         seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)


def uniform01(w: np.ndarray) -> np.ndarray:
    """(w + 0.5) / 2^32 in fp64: strictly inside (0, 1)."""
    return (np.asarray(w, np.uint32).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)


def normal(seed: int, tag: int, count: int, offset: int = 0) -> np.ndarray:
    """count N(0,1) fp64 draws, element e taken from Philox index (offset + e) // 4.

    Box-Muller on two pairs of uniforms per counter: words (0,1) give draws 0 and 1,
    words (2,3) give draws 2 and 3.
    """
    first = offset // 4
    last = (offset + count + 3) // 4
    idx = np.arange(first, last, dtype=np.uint64)
    w0, w1, w2, w3 = words(seed, tag, idx)
    u0, u1, u2, u3 = uniform01(w0), uniform01(w1), uniform01(w2), uniform01(w3)
    r0 = np.sqrt(-2.0 * np.log(u0))
    r1 = np.sqrt(-2.0 * np.log(u2))
    t0 = 2.0 * np.pi * u1
    t1 = 2.0 * np.pi * u3
    z = np.stack([r0 * np.cos(t0), r0 * np.sin(t0), r1 * np.cos(t1), r1 * np.sin(t1)], axis=1)
    z = z.reshape(-1)
    skip = offset - first * 4
    return z[skip:skip + count]


def uniform(seed: int, tag: int, count: int) -> np.ndarray:
    """count U(0,1) fp64 draws (one per Philox word)."""
    idx = np.arange((count + 3) // 4, dtype=np.uint64)
    w = np.stack(words(seed, tag, idx), axis=1).reshape(-1)[:count]
    return uniform01(w)


def randint(seed: int, tag: int, count: int, lo: int, hi: int) -> np.ndarray:
    """count integers uniform in [lo, hi] (inclusive), by scaling a U(0,1) draw."""
    u = uniform(seed, tag, count)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


def permutation(seed: int, tag: int, n: int) -> np.ndarray:
    """A uniformly random permutation of 0..n-1 (sort of random 64-bit keys)."""
    idx = np.arange(n, dtype=np.uint64)
    w0, w1, _, _ = words(seed, tag, idx)
    key = (w0.astype(np.uint64) << np.uint64(32)) | w1.astype(np.uint64)
    return np.lexsort((idx, key)).astype(np.int64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values straight to bf16 (nearest, ties to even); uint16 bit patterns.

    Rounds the fp64 bit pattern at the 7th fraction bit (no intermediate fp32, so
    no double rounding), then re-biases the exponent.  Inputs must be zero or of
    magnitude inside the bf16 normal range, which holds for the workloads here.
    """
    x = np.asarray(x, np.float64)
    ax = np.abs(x)
    if np.any((ax != 0) & ((ax < 2.0 ** -126) | (ax >= 2.0 ** 127))) or np.any(~np.isfinite(x)):
        raise ValueError("value outside the bf16 normal range")
    b = x.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + (np.uint64((1 << 44) - 1) + lsb)) >> np.uint64(45)     # sign|exp11|frac7
    sign = (r >> np.uint64(18)) & np.uint64(1)
    e11 = (r >> np.uint64(7)) & np.uint64(0x7FF)
    frac = r & np.uint64(0x7F)
    e8 = (e11.astype(np.int64) - 1023 + 127)
    out = (sign << np.uint64(15)) | (e8.astype(np.uint64) << np.uint64(7)) | frac
    out = np.where(ax == 0, sign << np.uint64(15), out)
    return out.astype(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
