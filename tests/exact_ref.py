"""Exact rational helpers used to pin the oracle (tests only).

Everything here works on ``fractions.Fraction`` and Python integers, so it
shares no floating-point arithmetic with the oracle and none of its code.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F16_MAX_MID = Fraction(65520)  # halfway between 65504 and 2**16: ties round up to inf


def frac_of_f16(h) -> Fraction:
    return Fraction(float(np.float16(h)))


def round_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def f16_round_exact(v: Fraction) -> float:
    """binary16 round-to-nearest-even of an exact rational; returns a Python
    float holding the fp16 value (inf on overflow)."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = -v if v < 0 else v
    if a >= F16_MAX_MID:
        return sign * float("inf")
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -14) - 10)
    n = round_half_even(a / quantum)
    return sign * float(n * quantum)


def brute_force_level(wv: Fraction, d: Fraction, z: int, max_int: int = 15) -> int:
    """Code q in 0..max_int whose level (q - z) d is nearest to wv; on an
    exact tie the level with (q - z) even wins."""
    best = None
    for q in range(max_int + 1):
        dist = abs(wv - (q - z) * d)
        key = (dist, (q - z) % 2)
        if best is None or key < best[0]:
            best = (key, q)
    return best[1]


def brute_force_zero(mn: Fraction, d: Fraction, max_int: int = 15) -> int:
    """Zero z in 0..max_int nearest to -mn / d; ties go to the even z."""
    best = None
    for z in range(max_int + 1):
        dist = abs(-mn / d - z)
        key = (dist, z % 2)
        if best is None or key < best[0]:
            best = (key, z)
    return best[1]


def exact_group_quant(row_vals, g: int, max_int: int = 15):
    """Independent exact quantization of one row of W' values (fp16, given as
    floats) with levels 0..max_int: returns (steps, zeros, codes) with steps
    as Python floats."""
    vals = [Fraction(float(v)) for v in row_vals]
    steps, zeros, codes = [], [], []
    for j in range(0, len(vals), g):
        grp = vals[j:j + g]
        mx, mn = max(grp), min(grp)
        r = max(mx - mn, Fraction(1, 2 ** 16))
        d = Fraction(f16_round_exact(r / max_int))
        z = brute_force_zero(mn, d, max_int)
        steps.append(float(d))
        zeros.append(z)
        codes.extend(brute_force_level(v, d, z, max_int) for v in grp)
    return steps, zeros, codes


def exact_loss(w16, x16, s16, g: int) -> Fraction:
    """Exact rational search loss for tiny shapes: fake-quantize W*s with the
    exact helpers above, then sum_{t,n} (sum_k ((q-z) d / s_k - w_nk) x_tk)^2."""
    w = np.asarray(w16, np.float16)
    x = np.asarray(x16, np.float16)
    s = np.asarray(s16, np.float16)
    n, k = w.shape
    m = x.shape[0]
    sf = [Fraction(float(v)) for v in s]
    total = Fraction(0)
    dws = []
    for r in range(n):
        wp = [f16_round_exact(Fraction(float(w[r, c])) * sf[c]) for c in range(k)]
        steps, zeros, codes = exact_group_quant(wp, g)
        dw = []
        for c in range(k):
            j = c // g
            deq = (codes[c] - zeros[j]) * Fraction(steps[j])
            dw.append(deq / sf[c] - Fraction(float(w[r, c])))
        dws.append(dw)
    for t in range(m):
        xt = [Fraction(float(v)) for v in x[t]]
        for r in range(n):
            e = sum(dws[r][c] * xt[c] for c in range(k))
            total += e * e
    return total
