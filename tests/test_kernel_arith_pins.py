"""CPU pins of arithmetic choices the GPU kernels rely on (not of the oracle).

1. The per-element code: the kernels compute RNE(w / D) for fp16 w and an
   fp16 step D > 0 as rintf(t2) with rd = fp32(1 / D) correctly rounded,
   t1 = fp32(w * rd), r = fma(-t1, D, w), t2 = fma(r, rd, t1) (awq_common.h,
   rne_quot).  This test emulates those fp32 operations exactly and checks,
   for every pair of finite fp16 values with D > 0 and |w / D| <= 16, that the
   result equals the exact round-half-to-even of the rational w / D (computed
   with integers).  The codes' clamp covers |w / D| > 16 (z <= 15, so any
   rounding of a larger quotient clamps to the same code).

2. The candidate scales s = fp16_rn(a^alpha): the GPU takes pow in float64
   on the device, the oracle numpy's; both are within a few float64 ulps of the
   exact power, so they round to the same fp16 unless the float64 power lies
   within that distance of an fp16 rounding boundary.  On the workloads'
   calibration statistics every power is far from a boundary.
"""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O


def _f16_values():
    """Every finite fp16 value (both signs, zeros once) as float64, with its
    integer significand and exponent: value = sig * 2^exp exactly."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)            # +0 .. max finite
    e = (bits >> 10).astype(np.int64)
    f = (bits & 0x3FF).astype(np.int64)
    sig = np.where(e == 0, f, f | 0x400)
    exp = np.where(e == 0, -24, e - 25)
    return bits, sig, exp


def _fp32_round_exact(hi, lo):
    """RNE to fp32 of the exact value hi + lo, where hi = fl64(hi + lo) and lo is
    the exact float64 error term (TwoSum).  Every fp32 rounding boundary (a
    midpoint between neighbouring fp32 values) is a float64 value, so no
    boundary lies strictly between hi and the exact sum: fl32 of the sum is
    fl32(hi) unless hi is itself a midpoint, where the sign of lo decides."""
    c = hi.astype(np.float32)
    c64 = c.astype(np.float64)
    up = np.nextafter(c, np.float32(np.inf), dtype=np.float32)
    dn = np.nextafter(c, np.float32(-np.inf), dtype=np.float32)
    out = np.where((hi == (c64 + up.astype(np.float64)) / 2.0) & (lo > 0), up, c)
    out = np.where((hi == (c64 + dn.astype(np.float64)) / 2.0) & (lo < 0), dn, out)
    return out


def _fma32(a, b, c):
    """fp32 fma(a, b, c) emulated exactly: a*b is exact in float64 (24 x 24
    bits), the sum with c is split by TwoSum into an exact float64 pair."""
    p = a.astype(np.float64) * b.astype(np.float64)
    cc = c.astype(np.float64)
    s = p + cc
    bb = s - p
    err = (p - (s - bb)) + (cc - bb)
    return _fp32_round_exact(s, err)


def _rne_exact(wsig, wexp, dsig, dexp):
    """Round half to even of (wsig 2^wexp) / (dsig 2^dexp) with integers."""
    sh = wexp - dexp
    num = np.where(sh >= 0, np.abs(wsig) << np.maximum(sh, 0), np.abs(wsig))
    den = np.where(sh >= 0, dsig, dsig << np.maximum(-sh, 0))
    q = num // den
    rem = num - q * den
    twice = 2 * rem
    up = (twice > den) | ((twice == den) & (q % 2 == 1))
    q = q + up.astype(np.int64)
    return np.where(wsig < 0, -q, q)


def test_rne_quot_exhaustive_fp16_pairs():
    bits, sig, exp = _f16_values()
    val = np.ldexp(sig.astype(np.float64), exp.astype(np.int64))
    # signed w: every finite fp16 (the negative zero behaves as +0)
    w_all = np.concatenate([val, -val[1:]])
    wsig_all = np.concatenate([sig, -sig[1:]])
    wexp_all = np.concatenate([exp, exp[1:]])
    order = np.argsort(w_all)
    w_all, wsig_all, wexp_all = w_all[order], wsig_all[order], wexp_all[order]
    w32_all = w_all.astype(np.float32)
    checked = 0
    for di in range(1, len(val)):                      # every positive finite D
        d = val[di]
        lo = np.searchsorted(w_all, -16.0 * d, side="left")
        hi = np.searchsorted(w_all, 16.0 * d, side="right")
        w32 = w32_all[lo:hi]
        d32 = np.float32(d)
        rd = np.float32(1.0) / d32                    # IEEE division: correctly rounded
        t1 = (w32 * rd).astype(np.float32)
        r = _fma32(-t1, np.full_like(t1, d32), w32)
        t2 = _fma32(r, np.full_like(t1, rd), t1)
        got = np.rint(t2).astype(np.int64)            # rintf: ties to even
        want = _rne_exact(wsig_all[lo:hi], wexp_all[lo:hi], sig[di], exp[di])
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (float(d), float(w_all[lo + bad[0]]), int(got[bad[0]]), int(want[bad[0]]))
        checked += hi - lo
    assert checked == 1_248_976_895          # every pair with |w / D| <= 16


def test_pow_candidates_far_from_fp16_boundaries():
    # calibration statistics of the workloads' inputs (Llama-3-8B-shaped with
    # 1 % x20 outliers, Llama-3-70B-shaped with 0.5 % x30), every grid alpha
    worst = np.inf
    for cfg, k, frac, mult in ((3, 4096, 0.01, 20.0), (3, 14336, 0.01, 20.0), (4, 8192, 0.005, 30.0),
                               (4, 28672, 0.005, 30.0), (1, 4096, 0.01, 20.0)):
        ch = S.outlier_channels(k, frac, S.seed_of(cfg, 0, 7, 3))
        a = O.calib_stats(S.activations(128, k, S.seed_of(cfg, 0, 7, 1), ch, mult))
        for alpha in O.alpha_grid(20)[1:]:
            p = np.power(a, alpha)
            p = np.maximum(p, 2.0 ** -14)
            h = p.astype(np.float16).astype(np.float64)
            # the rounding boundary nearest p: the midpoint between h and its
            # neighbour on p's side
            nb = np.where(p >= h, np.nextafter(h.astype(np.float16), np.float16(np.inf)),
                          np.nextafter(h.astype(np.float16), np.float16(-np.inf))).astype(np.float64)
            mid = (h + nb) / 2.0
            ulps = np.abs(p - mid) / np.spacing(p)
            worst = min(worst, float(ulps.min()))
    # any two float64 pows within 4 ulps of the exact power agree on fp16
    assert worst > 8.0, worst
