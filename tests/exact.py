"""Exact reference arithmetic used to pin the oracle.

These helpers reach the same plain definitions as the oracle by a different
route: integer arithmetic on fp16 values scaled by 2^24 (every finite binary16
value is an integer multiple of 2^-24) and Python ``Fraction``s, with numpy's
own float16 conversion as the codec.  Nothing here calls the oracle.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

UNIT = 1 << 24  # binary16 values are integer multiples of 2^-24


def f16_units(bits) -> np.ndarray:
    """binary16 bit patterns -> exact int64 value * 2^24 (finite inputs)."""
    v = np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
    u = v * float(UNIT)
    assert np.all(np.isfinite(u)) and np.all(u == np.round(u))
    return u.astype(np.int64)


def rne_div(X: np.ndarray, S) -> np.ndarray:
    """Round-half-even of the exact rational X / S for integer arrays, S > 0."""
    X = np.asarray(X, np.int64)
    S = np.asarray(S, np.int64)
    q0 = np.floor_divide(X, S)
    r2 = 2 * (X - q0 * S)  # 0 <= r2 < 2S
    up = (r2 > S) | ((r2 == S) & (q0 % 2 != 0))
    return q0 + up.astype(np.int64)


def fraction_to_f16_bits(x: Fraction) -> int:
    """Exact rational -> binary16 bits with round-to-nearest-even (finite range)."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    quantum = Fraction(2) ** (e - 10)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= 65520:
        return sign | 0x7C00
    if v < Fraction(1, 1 << 14):
        return sign | int(v * UNIT)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    frac = int(v / Fraction(2) ** (e - 10)) - 1024
    return sign | ((e + 15) << 10) | frac


def bits_to_fraction(b: int) -> Fraction:
    return Fraction(int(f16_units(np.array([b], np.uint16))[0]), UNIT)


def quant_exact(v_bits, qmax: int):
    """Brute-force symmetric quantizer: (q int64[L], s_bits) from exact rationals."""
    v_bits = np.asarray(v_bits, np.uint16).ravel()
    X = f16_units(v_bits)
    a = int(np.max(np.abs(X)))
    s_bits = fraction_to_f16_bits(Fraction(a, UNIT) / qmax)
    S = int(f16_units(np.array([s_bits], np.uint16))[0])
    if S == 0:
        return np.zeros(v_bits.size, np.int64), s_bits
    q = np.clip(rne_div(X, S), -qmax, qmax)
    return q, s_bits


def sign_extend4(nib: np.ndarray) -> np.ndarray:
    """4-bit two's complement -> int, via the xor-8 identity."""
    nib = np.asarray(nib, np.int64) & 0xF
    return (nib ^ 8) - 8


def unpack4_words(q4: np.ndarray) -> np.ndarray:
    """Packed 4-bit rows uint8 [N][K/2] -> int64 [N][K], read word by word: the
    little-endian 32-bit word d of a row holds k = 8d .. 8d+7, the even k
    (8d + 2i) in the four nibbles of its low half-word and the odd k
    (8d + 2i + 1) in those of its high half-word, nibble i at bits 4i."""
    b = np.asarray(q4, np.int64)
    N, KB = b.shape
    words = b.reshape(N, KB // 4, 4)
    lo16 = words[:, :, 0] | (words[:, :, 1] << 8)
    hi16 = words[:, :, 2] | (words[:, :, 3] << 8)
    out = np.empty((N, KB // 4, 8), np.int64)
    for i in range(4):
        out[:, :, 2 * i] = sign_extend4(lo16 >> (4 * i))
        out[:, :, 2 * i + 1] = sign_extend4(hi16 >> (4 * i))
    return out.reshape(N, 2 * KB)

