"""Exact rational brute force for tiny cases (pins the float64 oracle).

TEST INFRASTRUCTURE ONLY. Written independently of ``oracle.c``: the fp4
values come from the literal E2M1 value table of the OCP Microscaling (MX)
format specification, the scale value from the E4M3 bit fields via exact
fractions, and sums are exact (``fractions.Fraction``), so any dropped term,
sign, index or operand swap in the float64 oracle shows up as a mismatch
larger than its rounding bound.
"""
from __future__ import annotations

from fractions import Fraction

# OCP MX v1.0, FP4 (E2M1): magnitudes for the 3-bit magnitude field 0..7
E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e2m1(code: int) -> Fraction:
    mag = E2M1_MAG[code & 7]
    return -mag if code & 8 else mag


def e4m3(byte: int):
    """Exact value of an E4M3FN byte, or None for NaN."""
    s, e, m = (byte >> 7) & 1, (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        v = Fraction(m, 8) / 64
    else:
        v = Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))
    return -v if s else v


def bf16(bits: int) -> Fraction:
    import struct
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    return Fraction(f)


def weight(codes, scales, n: int, k: int) -> Fraction:
    """W[n][k] from the plain layout: byte k//2 of row n, low nibble for even k."""
    b = int(codes[n][k // 2])
    c = (b & 15) if k % 2 == 0 else (b >> 4)
    return e2m1(c) * e4m3(int(scales[n][k // 32]))


def matvec(codes, scales, x) -> list:
    """Exact W x for rational x (a list of Fractions)."""
    N = len(codes)
    K = len(codes[0]) * 2
    out = []
    for n in range(N):
        acc = Fraction(0)
        for k in range(K):
            acc += weight(codes, scales, n, k) * x[k]
        out.append(acc)
    return out


def abs_matvec(codes, scales, x) -> list:
    """sum_k |W[n][k] x[k]| (for rounding bounds)."""
    N = len(codes)
    K = len(codes[0]) * 2
    return [sum(abs(weight(codes, scales, n, k) * x[k]) for k in range(K)) for n in range(N)]
