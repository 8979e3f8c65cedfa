"""Quantizer inputs that sit exactly on rounding ties, with their expected
answers derived in exact rational arithmetic.

The contract rounds a quotient to an integer half to even (the MinMax code
and zero point of the GreenBit.AI article "只需单卡RTX 3090，低比特量化训练就能实现
LLaMA-3 8B全参微调", section 模型量化, and the int8 code of double quantization,
"QLoRA技术在量化微调中的应用", section QLoRA技术原理), and gives an NF4 value
that lies exactly on a midpoint between two levels the lower code.  Random
inputs almost never land on such a tie, so these builders place every value on
one: all values are small multiples of a power of two, so every fp32 quotient
the quantizer forms is exact and only the tie rule decides the result.

The expected integers are computed here with ``fractions.Fraction`` and an
explicit "nearest integer, ties to the even one" rule, not with any rounding
routine of numpy or of the oracle.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32


def round_half_even(t: Fraction) -> int:
    """Nearest integer to t; at an exact half, the even one."""
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def minmax_tie_groups(bits: int, group: int):
    """Groups of one row each whose scale is exactly 2^-4 and whose codes or
    zero point land on half-integers.

    Returns (W f32[n, group], expect dict with codes u8[n, group], scales
    f32[n, 1], zeros u8[n, 1]).  Group kinds:
      * range [0, Qmax/16]: w = (j + 1/2)/16 for every j (code ties, z = 0);
      * range [-Qmax/16, 0]: w = -(j + 1/2)/16 (negative code ties, z = Qmax);
      * range [-(j + 1/2)/16, (Qmax - j - 1/2)/16] for j = 0..Qmax-1: a zero
        point tie (z = round_half_even(j + 1/2)) plus the code ties that
        shift with it.
    """
    qmax = (1 << bits) - 1
    s = Fraction(1, 16)
    rows = []
    # value lists per group: the two ends of the range first, then the ties
    for sign in (+1, -1):
        ends = [Fraction(0), sign * qmax * s]
        ties = [sign * (j + Fraction(1, 2)) * s for j in range(qmax)]
        rows.append(ends + ties)
    for j in range(qmax):
        lo = -(j + Fraction(1, 2)) * s
        hi = lo + qmax * s
        ties = [lo + (i + Fraction(1, 2)) * s for i in range(qmax)]  # integer multiples of s
        halves = [Fraction(2 * i + 1, 32) for i in range(-qmax, qmax) if lo <= Fraction(2 * i + 1, 32) <= hi]
        rows.append([lo, hi] + ties + halves)
    W = np.zeros((len(rows), group), dtype=F32)
    codes = np.zeros((len(rows), group), dtype=np.uint8)
    zeros = np.zeros((len(rows), 1), dtype=np.uint8)
    for r, vals in enumerate(rows):
        lo = min(Fraction(0), min(vals))
        hi = max(Fraction(0), max(vals))
        assert (hi - lo) / qmax == s
        z = min(max(round_half_even(-lo / s), 0), qmax)
        zeros[r, 0] = z
        full = [vals[i % len(vals)] for i in range(group)]
        for i, v in enumerate(full):
            W[r, i] = F32(float(v))
            assert Fraction(float(W[r, i])) == v  # exact in fp32
            codes[r, i] = min(max(round_half_even(v / s) + z, 0), qmax)
    scales = np.full((len(rows), 1), F32(1.0 / 16.0), dtype=F32)
    return W, {"codes": codes, "scales": scales, "zeros": zeros}


def dq_tie_absmax(nblocks: int = 512, block: int = 256):
    """Absmax values whose double-quantization quotients are exact ties.

    Run r of ``block`` values has maximum 127 * 2^-(10 + r), so c2 = 2^-(10+r)
    exactly, and its other values are (j + 1/2) * c2 for j cycling through
    0..126 (plus some exact integers j * c2).  Returns (absmax f32[nblocks],
    expect dict with absmax_q i8[nblocks], absmax_scale f32[runs])."""
    runs = -(-nblocks // block)
    a = np.zeros(nblocks, dtype=F32)
    q2 = np.zeros(nblocks, dtype=np.int8)
    c2s = np.zeros(runs, dtype=F32)
    for r in range(runs):
        c2 = Fraction(1, 2 ** (10 + r))
        c2s[r] = F32(float(c2))
        for i in range(min(block, nblocks - r * block)):
            if i == 0:
                t = Fraction(127)
            elif i % 3 == 0:
                t = Fraction((7 * i) % 128)
            else:
                t = Fraction((5 * i) % 127) + Fraction(1, 2)
            a[r * block + i] = F32(float(t * c2))
            assert Fraction(float(a[r * block + i])) == t * c2
            q2[r * block + i] = min(max(round_half_even(t), 0), 127)
    return a, {"absmax_q": q2, "absmax_scale": c2s}


def nf4_midpoint_blocks(mids: np.ndarray, scale_exp: int = 0):
    """Blocks of 64 whose absmax is 2^scale_exp (an element equal to it) and
    whose other values put x = w / absmax exactly on each midpoint m_i, one
    fp32 step below and one above.  Returns (W f32[rows, 64], xs f32[rows,
    64]) with xs the exact quotients."""
    mids = np.asarray(mids, dtype=F32)
    pts = np.concatenate([mids, np.nextafter(mids, F32(-2)), np.nextafter(mids, F32(2)),
                          np.array([-1.0, 0.0, 1.0], dtype=F32)]).astype(F32)
    per = 63
    nrows = -(-pts.size // per)
    body = np.resize(pts, nrows * per).reshape(nrows, per)
    xs = np.concatenate([np.ones((nrows, 1), dtype=F32), body], axis=1).astype(F32)
    W = (xs.astype(np.float64) * 2.0 ** scale_exp).astype(F32)
    assert np.array_equal(W.astype(np.float64), xs.astype(np.float64) * 2.0 ** scale_exp)
    return W, xs


def nf4_power_of_two_blocks(rows: int = 128, k: int = 256, seed: int = 17):
    """Blocks of 64 with entries in {-a, 0, a}, a = q * 2^-(3 + r) with q an
    integer in 1..127 that differs from block to block and r the index of the
    block's run of 256 blocks; every run holds a block with q = 127.  Such a
    weight is exact in bf16, its codes are 0, 7 and 15, and double
    quantization reproduces every a exactly (c2 = 2^-(3+r), q2 = q).
    Returns W f32[rows, k]."""
    rng = np.random.default_rng(seed)
    nb = rows * k // 64
    W = np.zeros((nb, 64), dtype=F32)
    for b in range(nb):
        r, i = divmod(b, 256)
        q = 1 + (37 * i + 11 * r) % 127
        a = q * 2.0 ** -(3 + r)
        pat = rng.integers(-1, 2, size=64)
        pat[rng.integers(0, 64)] = 1 if rng.random() < 0.5 else -1
        W[b] = (pat * a).astype(F32)
    return W.reshape(rows, k)


def offset_tie_absmax(runs=2):
    """Absmax values in adjacent pairs 0.5 + t, 0.5 - t (each pair sums to 1
    exactly, so the mean is 0.5), t = (j + 1/2) / 1024 or j / 1024 with
    max t = 127/1024 in every run of 256: c2 = 2^-10 and d / c2 = +-(j + 1/2)."""
    a, want = [], []
    for r in range(runs):
        for p in range(128):
            t = Fraction(127, 1024) if p == 0 else (Fraction(2 * ((5 * p) % 127) + 1, 2048) if p % 2 else Fraction((3 * p) % 128, 1024))
            for sgn in (1, -1):
                a.append(F32(float(Fraction(1, 2) + sgn * t)))
                assert Fraction(float(a[-1])) == Fraction(1, 2) + sgn * t
                want.append(round_half_even(sgn * t * 1024))
    return np.array(a, dtype=F32), np.array(want, dtype=np.int8)
