"""Brute-force checkers for tiny inputs, written independently of the oracle.

They restate the definitions in the most literal way available (rank counts,
bit strings, exact rationals) so that a slip in the oracle's arithmetic (a
wrong comparison, a dropped term, a wrong bit order) shows up as a mismatch.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np


def f32(x) -> np.float32:
    return np.float32(x)


def kept_by_rank(acc: np.ndarray, lo: int, hi: int, k: int) -> List[int]:
    """Indices i in [lo, hi) whose rank (by |acc| desc, then index asc) < k.

    O(m^2) rank count: rank(i) = #{j : |a_j| > |a_i| or (|a_j| == |a_i| and j < i)}.
    """
    out = []
    mags = [abs(float(acc[i])) for i in range(lo, hi)]
    for a in range(hi - lo):
        rank = 0
        for b in range(hi - lo):
            if mags[b] > mags[a] or (mags[b] == mags[a] and b < a):
                rank += 1
        if rank < k:
            out.append(lo + a)
    return out


def ceil_frac(num: int, den: int) -> int:
    return -((-num) // den)


def rice_bits_string(positions: Sequence[int], b: int) -> str:
    """The Rice bit string of a position list, one character per bit."""
    out = []
    prev = -1
    for p in positions:
        z = p - prev - 1
        prev = p
        q, rem = divmod(z, 1 << b)
        out.append("1" * q + "0" + "".join("1" if (rem >> i) & 1 else "0" for i in range(b)))
    return "".join(out)


def pack_bits(bits: str) -> List[int]:
    """Pack a bit string into 32-bit words, string character i -> bit i % 32 of word i // 32."""
    words = [0] * ((len(bits) + 31) // 32)
    for i, ch in enumerate(bits):
        if ch == "1":
            words[i // 32] |= 1 << (i % 32)
    return words


def parse_rice(bits: str, count: int, b: int) -> Tuple[List[int], int]:
    """Inverse of rice_bits_string on a string; returns (positions, bits used)."""
    pos, prev, i = [], -1, 0
    for _ in range(count):
        q = 0
        while bits[i] == "1":
            q += 1
            i += 1
        i += 1
        rem = sum((1 << j) for j in range(b) if bits[i + j] == "1")
        i += b
        prev = prev + 1 + q * (1 << b) + rem
        pos.append(prev)
    return pos, i


def exact_mean(values: Sequence[float]) -> Fraction:
    vals = [Fraction(float(v)) for v in values]
    return sum(vals, Fraction(0)) / len(vals)


def ulp32(x: float) -> float:
    x = abs(np.float32(x))
    return float(np.spacing(x)) if x > 0 else float(np.finfo(np.float32).smallest_subnormal)
