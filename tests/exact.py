"""Exact reference arithmetic used by the oracle's pins.

Everything here is computed by a different method from the oracle's: rational
arithmetic (``fractions``), 50-digit decimal transcendental functions
(``decimal``), integer bit manipulation and library routines (numpy, the
Python sort).  Nothing here is imported by the oracle or the GPU library.
"""
from __future__ import annotations

import decimal
import functools
import struct
from fractions import Fraction

import numpy as np

_CTX = decimal.Context(prec=50)


def f32_bits(v) -> int:
    return int(np.array(v, np.float32).view(np.uint32))


def round_f32(fr: Fraction) -> np.float32:
    """Correct rounding of an exact rational to binary32, ties to even."""
    if fr == 0:
        return np.float32(0.0)
    c = np.float32(float(fr))
    if not np.isfinite(c):
        return c
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    cands = [v for v in cands if np.isfinite(v)]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), f32_bits(v) & 1))


def dec_score(kind: str, logit: float) -> Fraction:
    """sigmoid or sqrt(softplus) of a logit, to 50 significant digits."""
    with decimal.localcontext(_CTX):
        l = decimal.Decimal(float(logit))
        if kind == "sigmoid":
            v = 1 / (1 + (-l).exp())
        else:
            u = l.exp() if l <= 0 else (-l).exp()
            lp = (1 + u).ln() if u > decimal.Decimal("1e-20") else u - u * u / 2
            sp = lp if l <= 0 else l + lp
            v = sp.sqrt()
        return Fraction(v)


@functools.lru_cache(maxsize=1 << 16)
def score_f32(kind: str, logit: float) -> np.float32:
    return round_f32(dec_score(kind, logit))


def bf16_round_bits(v: float) -> int:
    """Round a double to bf16 (ties to even) by integer arithmetic on its bits."""
    u = struct.unpack("<Q", struct.pack("<d", float(v)))[0]
    sign = (u >> 63) & 1
    ex = (u >> 52) & 0x7FF
    man = u & ((1 << 52) - 1)
    if ex == 0x7FF:
        return (sign << 15) | (0x7FC0 if man else 0x7F80)
    if ex == 0 and man == 0:
        return sign << 15
    # value = M * 2^E with integer M
    if ex == 0:
        M, E = man, -1074
    else:
        M, E = man | (1 << 52), ex - 1075
    # bf16 grid at this magnitude: quantum 2^(e_lead - 7) with e_lead >= -126,
    # i.e. quantum >= 2^-133.
    e_lead = M.bit_length() - 1 + E
    q = max(e_lead - 7, -133)
    shift = q - E
    if shift > 0:
        n, rem = divmod(M, 1 << shift)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (n & 1)):
            n += 1
    else:
        n = M << (-shift)
    # value now n * 2^q
    if n == 0:
        return sign << 15
    val = Fraction(n) * Fraction(2) ** q
    if val >= Fraction(2) ** 128:
        return (sign << 15) | 0x7F80
    f = np.float32(float(val))  # exact: n has <= 8 significant bits
    return (sign << 15) | ((f32_bits(f) >> 16) & 0x7FFF)


def bf16_round_array(a: np.ndarray) -> np.ndarray:
    """Vector version: returns the rounded values as float64."""
    out = np.empty(a.shape, np.float64)
    flat, of = a.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        b = bf16_round_bits(float(v))
        of[i] = float(np.array(b << 16, np.uint32).view(np.float32))
    return out


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_q8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int8 blocks of 32 along the last axis times their fp16 scale (numpy float16)."""
    sc = s.view(np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(sc, 32, axis=-1)


def as_f64(arr, fmt: str) -> np.ndarray:
    if isinstance(arr, tuple):
        return dequant_q8(*arr)
    if fmt == "f32":
        return arr.astype(np.float64)
    return widen_bf16(arr)
