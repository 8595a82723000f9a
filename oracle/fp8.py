"""Oracle 8-bit float (E4M3, the OCP "fn" variant) for a quantised KV pool.
Test infrastructure only.

The pages name quantisation as the way to shrink the cache when block
management has nothing left to save, at a cost in accuracy ("第 6 章 缓存管理",
section "缓存的边界"), and list the cache's element type among the things the
paged kernel must follow ("vLLM：把 KV 缓存当成虚拟内存", the paragraph on
variants).  They fix no format; the format here is E4M3 as the OCP 8-bit
floating-point specification defines it:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0: subnormal, value = (-1)^s * m/8 * 2^-6 (smallest 2^-9);
* otherwise value = (-1)^s * (1 + m/8) * 2^(e-7), largest 448 (e = 15, m = 6);
* e = 15, m = 7 is NaN (both signs); there is no infinity.

Quantisation of a K or V element x with per-pool scale c (stored value
approximates x / c): y = float32(x * float32(1 / c)) in float32 arithmetic,
clamped to [-448, 448], then rounded to the nearest E4M3 value, ties to the
even mantissa; NaN stays NaN.  Dequantisation: value(code) * c.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 15 and m == 7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALUES = e4m3_values()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(y: np.ndarray) -> np.ndarray:
    """float32 values already clamped to [-448, 448] (or NaN) -> uint8 codes,
    round to nearest, ties to even mantissa.  Done by comparison with the
    table of finite non-negative values: the nearest one wins, and on a tie
    the one with the even code (even mantissa) wins."""
    y = np.asarray(y, dtype=np.float64)
    pos = _VALUES[:0x7F]                       # codes 0x00..0x7E, increasing
    a = np.abs(y)
    hi = np.searchsorted(pos, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, len(pos) - 1)
    lo = np.clip(hi - 1, 0, len(pos) - 1)
    d_lo = np.abs(a - pos[lo])
    d_hi = np.abs(pos[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """float32 K/V values -> E4M3 codes for a pool with the given scale."""
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):          # huge inputs overflow to +-inf, then saturate
        y = np.asarray(x, dtype=np.float32) * inv
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3(y)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    return decode_e4m3(codes) * float(scale)
