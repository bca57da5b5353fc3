"""Pure-Python brute-force checker for tiny SVQ cases.

TEST INFRASTRUCTURE ONLY (same import rule as ``svq_oracle``).  Written
independently of ``svq_oracle``: no numpy, no vectorised bit tricks; it
walks the bitstream one bit at a time and decodes fp16 by its IEEE
definition, following the code structure of the SAGE paper's Fig. 2 caption
(signs, direction index, quantized radius; 18 bits per 8 weights).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence


def fp16_value(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (finite values only)."""
    sign = -1 if (bits >> 15) & 1 else 1
    exp = (bits >> 10) & 0x1F
    frac = bits & 0x3FF
    if exp == 0x1F:
        raise ValueError("inf/nan not expected")
    if exp == 0:
        return sign * Fraction(frac, 1 << 24)  # subnormal: frac * 2**-24
    return sign * Fraction(1024 + frac, 1024) * (Fraction(2) ** (exp - 15))


def bf16_value(bits: int) -> Fraction:
    """Exact value of a bfloat16 bit pattern (finite values only)."""
    sign = -1 if (bits >> 15) & 1 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("inf/nan not expected")
    if exp == 0:
        return sign * Fraction(frac, 128) * (Fraction(2) ** -126)
    return sign * Fraction(128 + frac, 128) * (Fraction(2) ** (exp - 127))


def read_field(stream: Sequence[int], first_bit: int, nbits: int) -> int:
    """Read nbits starting at stream bit first_bit, LSB first."""
    v = 0
    for j in range(nbits):
        t = first_bit + j
        bit = (int(stream[t // 8]) >> (t % 8)) & 1
        v |= bit << j
    return v


def decode_dense(stream: Sequence[int], n: int, k: int, bd: int,
                 codebook: Sequence[Sequence[int]], radius: Sequence[int],
                 perm: Sequence[int]) -> List[List[Fraction]]:
    """Exact dense W[n][k] (input-channel order) as Fractions."""
    c_per_row = k // 8
    w = [[Fraction(0)] * k for _ in range(n)]
    for i in range(n):
        for c in range(c_per_row):
            g = i * c_per_row + c
            base = 18 * g
            signs = read_field(stream, base, 8)
            d = read_field(stream, base + 8, bd)
            r = read_field(stream, base + 8 + bd, 10 - bd)
            rad = fp16_value(radius[r])
            for lane in range(8):
                v = rad * fp16_value(codebook[d][lane])
                if (signs >> lane) & 1:
                    v = -v
                w[i][perm[8 * c + lane]] = v
    return w


def linear(stream, n, k, bd, codebook, radius, perm, x_bits_rows) -> List[List[Fraction]]:
    """Exact y[m][n] = sum_j W[i][j] x[m][j] with x given as bf16 bit patterns."""
    w = decode_dense(stream, n, k, bd, codebook, radius, perm)
    out = []
    for xrow in x_bits_rows:
        xv = [bf16_value(b) for b in xrow]
        out.append([sum((w[i][j] * xv[j] for j in range(k)), Fraction(0)) for i in range(n)])
    return out
