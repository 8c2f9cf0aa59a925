"""Storage formats of the oracle: bf16 and OCP fp8 e4m3fn, each rounded once.

Test infrastructure (see the package docstring): nothing in the product path
imports this module.

The group-reading wiki page "DeepSeek-V4 深度研究剖析" §8 keeps the KV cache in
BF16 and FP8; the workloads store compressed K/V as bf16, or as fp8 e4m3 with
one fp32 scale per 64 entries.  Both conversions here go from an exact float64
value to the format in a single round-to-nearest-even step, written from the
formats' definitions:

  bf16    1 sign, 8 exponent, 7 fraction bits (float32's upper half).
  e4m3fn  1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities; the
          only NaN is S.1111.111; largest finite 448; smallest normal 2^-6,
          subnormal quantum 2^-9.
  e2m1    (OCP MX FP4) 1 sign, 2 exponent (bias 1), 1 fraction bit; no
          infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _round_to_quantum(x: np.ndarray, min_exp: int, frac_bits: int) -> np.ndarray:
    """Round float64 x to the grid of a binary format with `frac_bits` fraction
    bits and smallest normal exponent `min_exp`, ties to even.  Exact: the
    quantum is a power of two, so x / q is exact and rint does the rounding."""
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)                    # |x| = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, min_exp)        # exponent of the binade (or subnormal range)
    q = np.ldexp(1.0, e - frac_bits)
    return np.rint(x / q) * q


def bf16_round_value(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of float64 x (ties to even), as float64."""
    return _round_to_quantum(x, -126, 7)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one rounding step."""
    v = bf16_round_value(x).astype(np.float32)     # exact: v is a bf16 value
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> e4m3fn codes (uint8): clamp to +-448, then round to nearest
    even.  The sign bit is the sign bit of x (a negative value that rounds to
    zero gives the code of -0)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(np.clip(x, -E4M3_MAX, E4M3_MAX))
    v = _round_to_quantum(a, -6, 3)                 # a representable e4m3 magnitude
    code = np.zeros(x.shape, dtype=np.uint8)
    nz = v > 0
    _, E = np.frexp(v[nz])
    e = E - 1                                       # v = 1.f * 2^e for normals
    sub = e < -6
    mant_sub = np.rint(v[nz] / 2.0 ** -9)           # subnormal: v = mant * 2^-9
    mant_norm = np.rint((v[nz] / np.ldexp(1.0, e) - 1.0) * 8.0)
    expf = np.where(sub, 0, e + 7)
    mant = np.where(sub, mant_sub, mant_norm)
    code[nz] = (expf.astype(np.int64) << 3 | mant.astype(np.int64)).astype(np.uint8)
    return code | (sign.astype(np.uint8) << 7)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """e4m3fn codes -> float64 (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    mag = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return s * mag


E2M1_MAX = 6.0


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> e2m1 codes (uint8 in 0..15): clamp to +-6, then round to
    nearest even (quantum 0.5 below 2, 1 in [2, 4), 2 in [4, 6]).  The sign
    bit is the sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(np.clip(x, -E2M1_MAX, E2M1_MAX))
    v = _round_to_quantum(a, 0, 1)                  # a representable e2m1 magnitude
    # magnitude -> 3-bit code: 0, 0.5, 1, 1.5 -> 2v; 2, 3 -> v + 2; 4, 6 -> 4 + v / 2
    mag = np.where(v < 2, 2 * v, np.where(v < 4, v + 2, 4 + v / 2)).astype(np.int64)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    """e2m1 codes -> float64."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    return s * np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
