"""Error bound of the GPU search loss against the float64 oracle, derived from
the arithmetic the search kernel uses (test infrastructure; uses the oracle).

The kernel forms, per element, c dW = ((q - z) D - W s) * (c / s) in fp32: the
two terms of the difference are exact fp32 values, so the difference, the
rounded reciprocal c / s and the product add at most three roundings,
relative 3 u (u = 2^-24).  It splits c dW into fp16 hi = rtz(c dW) and
lo = rtz(c dW - hi): each truncation loses less than one fp16 ulp (relative
2^-10), so hi + lo is within 2^-20 |c dW| of c dW, plus at most one fp16
subnormal ulp (2^-24 in the scaled domain, 2^-24 / c in dW) where lo falls
below the normal range.  The block factor is c = 2^(14 - e) with
max |W| of its 64 rows below 2^e, so 1 / c < 2 max|W| / 2^14 over all rows.

E = dW X^T is accumulated by v_mfma_f32_32x32x16_f16 over K in steps of 16
channels, hi and lo in separate MFMAs into the same fp32 accumulator: K / 8
accumulations per output, each adding a 16-product sum (products of fp16
values are exact in fp32).  Counting every accumulation and a summation depth
of 5 inside one MFMA as one rounding each gives, to first order,

    |E_gpu - E| <= gamma * sum_k |dW_nk X_tk| + beta * sum_k |X_tk|,
    gamma = (K / 8 + 5 + 3) u + 2^-20,   beta = 2^-24 * 2 max|W| / 2^14.

The float64 squares and sums of E add a relative 1e-12 at most.  With
D^2 = sum_{t,n} (gamma A_tn + beta B_t)^2, A_tn = sum_k |dW_nk X_tk|,
B_t = sum_k |X_tk|, Cauchy-Schwarz gives

    |L_gpu - L| <= 2 sqrt(L) D + D^2   (+ 1e-12 L).

The chosen index is then certain to match when the oracle's best and second
losses differ by more than the sum of their two bounds; below that the pair
is a near tie and the match is still asserted.
"""
from __future__ import annotations

import numpy as np

from oracle import awq_oracle as O

U = 2.0 ** -24


def gamma_of(k: int) -> float:
    return (k / 8 + 5 + 3) * U + 2.0 ** -20


def loss_bounds(w16, x16, a, g, n_grid, w_bit=4):
    """Per-alpha bound on |L_gpu - L_oracle| (inf where the oracle loss is not finite)."""
    w16 = np.asarray(w16)
    x = np.abs(np.asarray(x16, np.float16).astype(np.float64))
    k = w16.shape[1]
    gam = gamma_of(k)
    wmax = float(np.max(np.abs(w16[np.isfinite(w16)].astype(np.float64)))) if np.isfinite(w16).any() else 0.0
    beta = U * 2.0 * wmax / 2.0 ** 14
    bsum = x.sum(axis=1)                         # B_t
    n = w16.shape[0]
    max_int = (1 << w_bit) - 1
    out = np.full(n_grid, np.inf)
    for i, al in enumerate(O.alpha_grid(n_grid)):
        s = O.scale_candidate(a, al)
        wp, q, z, d16, bad, deq = O.fake_quantize(w16, s, g, max_int)
        if bad.any():
            continue
        dw = np.abs(deq / s.astype(np.float64)[None, :] - w16.astype(np.float64))
        amat = dw @ x.T                          # A_tn as [n, t]
        d = np.sqrt(np.sum((gam * amat + beta * bsum[None, :]) ** 2))
        out[i] = d
    return out


def check_losses(gpu_losses, oracle_losses, dnorm):
    """Assert |L_gpu - L| <= 2 sqrt(L) D + D^2 + 1e-12 L per finite alpha; return the
    largest observed |L_gpu - L| / L."""
    gl = np.asarray(gpu_losses, np.float64)
    ol = np.asarray(oracle_losses, np.float64)
    fin = np.isfinite(ol)
    assert np.array_equal(np.isfinite(gl), fin)
    worst = 0.0
    for i in np.flatnonzero(fin):
        bound = 2.0 * np.sqrt(ol[i]) * dnorm[i] + dnorm[i] ** 2 + 1e-12 * ol[i]
        assert abs(gl[i] - ol[i]) <= bound, (i, gl[i], ol[i], bound)
        if ol[i] > 0:
            worst = max(worst, abs(gl[i] - ol[i]) / ol[i])
    return worst


def gap_report(oracle_losses, dnorm):
    """(best, second, relative gap (L2 - L1) / L1, margin = (L2 - L1) / (bound1 + bound2))
    for the oracle's losses; margin > 1 means the index cannot flip."""
    ol = np.asarray(oracle_losses, np.float64)
    best = O.select_best(ol)
    fin = [i for i in np.flatnonzero(np.isfinite(ol)) if i != best]
    if best < 0 or not fin:
        return best, -1, np.inf, np.inf
    second = min(fin, key=lambda i: (ol[i], i))
    gap = ol[second] - ol[best]
    b1 = 2.0 * np.sqrt(ol[best]) * dnorm[best] + dnorm[best] ** 2
    b2 = 2.0 * np.sqrt(ol[second]) * dnorm[second] + dnorm[second] ** 2
    rel = gap / ol[best] if ol[best] > 0 else np.inf
    return best, int(second), float(rel), float(gap / (b1 + b2)) if b1 + b2 > 0 else np.inf
