"""Pins of the CPU oracle against facts fixed independently of it: exact
rational arithmetic, brute force over all 16 levels, closed forms, known-answer
groups, invariants and the special case that reduces to textbook RTN.

Runs on the CPU (no GPU marker)."""
from __future__ import annotations

import json
import pathlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as O
from tests import exact_ref as X
import synthetic as S

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- rounding


def test_fp16_rn_matches_exact_rounding():
    r = _rng(1)
    vals = list(r.standard_normal(4000) * 10.0 ** r.integers(-9, 6, 4000))
    # exact fp16 midpoints (ties) around many binades, incl. subnormals and overflow edge
    for e in range(-24, 16):
        for mant in (1, 3, 1023, 1025, 2047):
            vals.append(float((Fraction(mant) + Fraction(1, 2)) * Fraction(2) ** (e - 10)))
    vals += [65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26]
    got = O.fp16_rn(np.array(vals))
    for v, h in zip(vals, got):
        want = X.f16_round_exact(Fraction(v))
        assert float(h) == want or (np.isinf(want) and np.isinf(float(h))), (v, float(h), want)


# ---------------------------------------------------------------- a1 stats


def test_calib_stats_exact_integer_sum():
    x = S.activations(257, 96, seed=11, channels=np.array([3, 50]), mult=20.0)
    a = O.calib_stats(x)
    bits = x.view(np.uint16).astype(np.int64)
    # |x| * 2**24 as an exact integer from the fp16 bit pattern
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    ints = np.where(e == 0, m, (m | 0x400) << np.maximum(e - 1, 0))
    for k in range(x.shape[1]):
        s_exact = sum(int(v) for v in ints[:, k])
        want = Fraction(s_exact, 2 ** 24 * x.shape[0])
        assert a[k] == float(want), k     # correctly rounded exact mean


def test_calib_stats_closed_form():
    c = np.float16(0.3125)
    signs = np.where(_rng(2).random((64, 40)) < 0.5, -1.0, 1.0)
    x = (signs * float(c)).astype(np.float16)
    assert np.all(O.calib_stats(x) == float(c))


# ---------------------------------------------------------------- a2 candidates


def test_scale_candidates_special_values():
    a = np.array([4.0, 0.25, 16.0, 0.0, 1.0, 3.7, np.nan])
    s = O.scale_candidate(a, 0.5).astype(np.float64)
    assert s[0] == 2.0 and s[1] == 0.5 and s[2] == 4.0
    assert s[3] == 2.0 ** -14          # lower clamp
    assert s[4] == 1.0
    assert s[5] == X.f16_round_exact(Fraction(float(np.sqrt(3.7))))
    assert np.isnan(s[6])
    s0 = O.scale_candidate(a, 0.0).astype(np.float64)
    assert np.all(s0 == 1.0)            # x**0 = 1, also for 0 and NaN
    assert O.scale_candidate(np.array([16.0]), 0.25)[0] == 2.0
    assert np.array_equal(O.alpha_grid(20), np.arange(20) / 20.0)


# ---------------------------------------------------------------- a3 codes


def _random_wp(n, k, seed, sigma=0.02):
    return S.weights(n, k, sigma, seed)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_codes_brute_force_all_levels(g):
    wp = _random_wp(6, 2 * g, 100 + g)
    # add groups that do not span zero, a constant group, tiny and large values
    wp[0, :g] = np.abs(wp[0, :g]) + np.float16(0.5)
    wp[1, g:] = np.float16(-0.75)
    wp[2, :g] = (wp[2, :g].astype(np.float64) * 1e-3).astype(np.float16)
    wp[3, g:] = (wp[3, g:].astype(np.float64) * 3000).astype(np.float16)
    d16, z, bad = O.group_params(wp, g)
    q = O.quantize_codes(wp, d16, z, g, bad)
    assert not bad.any()
    for r in range(wp.shape[0]):
        steps, zeros, codes = X.exact_group_quant(wp[r], g)
        assert list(d16[r].astype(np.float64)) == steps, r
        assert list(z[r]) == zeros, r
        assert list(q[r]) == codes, r


def test_codes_exact_ties_round_to_even():
    # a group whose values sit exactly on half steps: w = (k + 1/2) * d
    d = np.float16(2.0 ** -7)
    g = 32
    levels = np.array([(i % 15) - 7 for i in range(g)], dtype=np.float64)
    wp = np.zeros((1, g), np.float16)
    wp[0, :] = (levels * float(d)).astype(np.float16)
    wp[0, 0] = np.float16(-7 * float(d))
    wp[0, 1] = np.float16(8 * float(d))   # range = 15 d exactly, so step = d, z = 7
    for i, h in enumerate((0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5)):
        wp[0, 2 + i] = np.float16(h * float(d))
    d16, z, bad = O.group_params(wp, g)
    q = O.quantize_codes(wp, d16, z, g, bad)
    assert float(d16[0, 0]) == float(d) and z[0, 0] == 7
    got = [int(q[0, 2 + i]) - 7 for i in range(7)]
    assert got == [0, 2, 2, 0, -2, -2, 6]


def test_known_answer_groups_golden():
    data = json.loads((GOLDEN / "known_answer_groups.json").read_text())
    g = data["g"]
    for case in data["cases"]:
        d0 = np.float16(case["step"])
        z0 = case["zero"]
        q0 = np.array(case["codes"], dtype=np.int64)
        wp = ((q0 - z0).astype(np.float64) * float(d0)).astype(np.float16)[None, :]
        d16, z, bad = O.group_params(wp, g)
        q = O.quantize_codes(wp, d16, z, g, bad)
        assert float(d16[0, 0]) == float(d0)
        assert z[0, 0] == z0
        assert list(q[0]) == list(q0)


@pytest.mark.parametrize("g", [32, 128])
def test_known_answer_random_groups(g):
    r = _rng(7 + g)
    n, ng = 8, 4
    d0 = (2.0 ** r.integers(-12, -3, (n, ng))).astype(np.float16)
    # at most 7 significant bits, so (q - z) * d0 (|q - z| <= 15) is exact in fp16
    d0 = (d0.astype(np.float64) * (1 + r.integers(0, 64, (n, ng)) / 64)).astype(np.float16)
    z0 = r.integers(0, 16, (n, ng))
    q0 = r.integers(0, 16, (n, ng, g))
    q0[:, :, 0] = 0
    q0[:, :, 1] = 15
    wp = ((q0 - z0[:, :, None]) * d0.astype(np.float64)[:, :, None]).reshape(n, ng * g).astype(np.float16)
    d16, z, bad = O.group_params(wp, g)
    q = O.quantize_codes(wp, d16, z, g, bad)
    assert np.array_equal(d16, d0)
    assert np.array_equal(z, z0)
    assert np.array_equal(q.reshape(n, ng, g), q0)


def test_invariants_error_bound():
    g = 128
    w = _random_wp(64, 512, 5)
    s = O.scale_candidate(O.calib_stats(S.activations(32, 512, 6, np.arange(0, 512, 50), 20.0)), 0.45)
    wp, q, z, d16, bad, deq = O.fake_quantize(w, s, g)
    assert np.all((z >= 0) & (z <= 15)) and np.all((q >= 0) & (q <= 15))
    assert np.all(d16.astype(np.float64) > 0)
    d = np.repeat(d16.astype(np.float64), g, axis=1)
    err = np.abs(wp.astype(np.float64) - deq)
    wg = O.group_view(wp.astype(np.float64), g)
    exact_d = np.repeat(np.maximum(wg.max(2) - wg.min(2), 2.0 ** -16) / 15.0, g, axis=1)
    assert np.all(err <= d / 2 + 15 * np.abs(exact_d - d) + 1e-300)
    unclamped = (np.rint(wp.astype(np.float64) / d) + np.repeat(z, g, axis=1) >= 0) & \
                (np.rint(wp.astype(np.float64) / d) + np.repeat(z, g, axis=1) <= 15)
    assert np.all(err[unclamped] <= d[unclamped] / 2)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_pack_roundtrip(g):
    w = _random_wp(5, 8 * g + 3 * g if g < 128 else 3 * g, 9)
    k = w.shape[1]
    qw, sc, qz, nbad = O.pack_int4(w, None, g)
    assert nbad == 0
    assert qw.shape == (5, k // 8) and sc.shape == (5, k // g) and qz.shape == (5, -(-k // (8 * g)))
    q, z = O.unpack_int4(qw, qz, k, g)
    _, q2, z2, d2, _, _ = O.fake_quantize(w, None, g)
    assert np.array_equal(q, q2) and np.array_equal(z, z2) and np.array_equal(sc, d2)
    # unused zero nibbles are zero
    ng = k // g
    if ng % 8:
        top = (qz[:, -1].astype(np.uint64) >> np.uint64(4 * (ng % 8)))
        assert np.all(top == 0)
    # nibble order: bits 4*(k%8) of word k/8 hold q[k]
    assert (int(qw[2, 1]) >> 12) & 0xF == q[2, 11]


def test_nonfinite_groups_marked():
    g = 32
    w = _random_wp(2, 64, 4)
    w[1, 40] = np.float16(np.inf)
    s = np.ones(64, np.float16)
    s[5] = np.float16(60000.0)       # pushes W'[.,5] past fp16 max when |w| > 1.1
    w[0, 5] = np.float16(2.0)
    qw, sc, qz, nbad = O.pack_int4(w, s, g)
    assert nbad == 2
    assert sc.view(np.uint16)[0, 0] == O.F16_NAN_BITS and sc.view(np.uint16)[1, 1] == O.F16_NAN_BITS
    q, z = O.unpack_int4(qw, qz, 64, g)
    assert np.all(q[0, :32] == 0) and z[0, 0] == 0 and np.all(q[1, 32:] == 0)
    assert np.isinf(O.search_loss(w, S.activations(3, 64, 1), s, g))


# ---------------------------------------------------------------- a3/a4 search


def test_loss_matches_exact_fractions():
    w = _random_wp(2, 32, 21)
    x = S.activations(3, 32, 22, np.array([4]), 20.0)
    a = O.calib_stats(x)
    for alpha in (0.0, 0.35, 0.95):
        s = O.scale_candidate(a, alpha)
        got = O.search_loss(w, x, s, 32)
        want = X.exact_loss(w, x, s, 32)
        assert abs(got - float(want)) <= 1e-12 * float(want), alpha


def _textbook_rtn_error(w16, x16, g, max_int=15):
    """Loop-based min-max asymmetric round-to-nearest quantizer (s = 1), written
    independently of the oracle with exact rationals; returns the output error
    sum of squares."""
    w = np.asarray(w16, np.float16)
    x = np.asarray(x16, np.float16)
    n, k = w.shape
    tot = Fraction(0)
    deq = [[None] * k for _ in range(n)]
    for r in range(n):
        for j in range(0, k, g):
            grp = [Fraction(float(v)) for v in w[r, j:j + g]]
            lo, hi = min(grp), max(grp)
            step = Fraction(X.f16_round_exact(max(hi - lo, Fraction(1, 2 ** 16)) / max_int))
            zero = min(max_int, max(0, X.round_half_even(-lo / step)))
            for c, v in enumerate(grp):
                code = min(max_int, max(0, X.round_half_even(v / step) + zero))
                deq[r][j + c] = (code - zero) * step
    for t in range(x.shape[0]):
        for r in range(n):
            e = sum((deq[r][c] - Fraction(float(w[r, c]))) * Fraction(float(x[t, c])) for c in range(k))
            tot += e * e
    return tot


def test_alpha0_is_plain_rtn():
    w = _random_wp(3, 64, 31)
    x = S.activations(4, 64, 32, np.array([1, 9]), 20.0)
    a = O.calib_stats(x)
    best, s16, inv, losses = O.search_scale(w, x, a, g=32, n_grid=4)
    want = _textbook_rtn_error(w, x, 32)
    assert abs(losses[0] - float(want)) <= 1e-12 * float(want)


def test_tie_break_constant_activations():
    w = _random_wp(16, 128, 41)
    x = np.where(_rng(42).random((8, 128)) < 0.5, -1.0, 1.0).astype(np.float16)
    a = O.calib_stats(x)
    assert np.all(a == 1.0)
    best, s16, inv, losses = O.search_scale(w, x, a, g=64, n_grid=20)
    assert np.all(losses == losses[0])
    assert best == 0
    assert np.all(s16.astype(np.float64) == 1.0) and np.all(inv.astype(np.float64) == 1.0)


def test_select_best_rules():
    assert O.select_best(np.array([3.0, 1.0, 1.0, 2.0])) == 1
    assert O.select_best(np.array([np.nan, np.inf, 5.0, 5.0])) == 2
    assert O.select_best(np.array([np.nan, np.inf])) == -1


def test_search_beats_rtn_with_outliers():
    w = _random_wp(64, 256, 51)
    x = S.activations(32, 256, 52, S.outlier_channels(256, 0.02, 53), 20.0)
    a = O.calib_stats(x)
    best, s16, inv, losses = O.search_scale(w, x, a, g=128, n_grid=20)
    assert best > 0 and losses[best] < losses[0]
    assert np.all(losses[best] <= losses)
    assert np.array_equal(s16, O.scale_candidate(a, best / 20.0))
    want_inv = [X.f16_round_exact(1 / Fraction(float(v))) for v in s16]
    assert list(inv.astype(np.float64)) == want_inv


def test_scaling_identity_before_quantization():
    w = _random_wp(8, 64, 61).astype(np.float64)
    xv = S.activations(1, 64, 62).astype(np.float64)[0]
    s = 2.0 ** _rng(63).uniform(-3, 3, 64)
    lhs = (w * s[None, :]) @ (xv / s)
    rhs = w @ xv
    assert np.max(np.abs(lhs - rhs)) <= 1e-15 * 64 * np.max(np.abs(w)) * np.max(np.abs(xv)) * 8


# ---------------------------------------------------------------- linear


def test_linear_ref_exact_small():
    g = 32
    w = _random_wp(3, 64, 71)
    x = S.activations(2, 64, 72)
    s = O.scale_candidate(O.calib_stats(S.activations(8, 64, 73, np.array([5]), 20.0)), 0.4)
    inv = O.fp16_rn(1.0 / s.astype(np.float64))
    qw, sc, qz, _ = O.pack_int4(w, s, g)
    y = O.linear_ref(x, qw, sc, qz, inv, 64, g)
    # exact: unpack bits by hand and sum rationals
    for t in range(2):
        for n in range(3):
            acc = Fraction(0)
            for c in range(64):
                code = (int(qw[n, c // 8]) >> (4 * (c % 8))) & 0xF
                j = c // g
                zero = (int(qz[n, j // 8]) >> (4 * (j % 8))) & 0xF
                acc += Fraction(float(x[t, c])) * Fraction(float(inv[c])) * (code - zero) * Fraction(float(sc[n, j]))
            assert abs(y[t, n] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc)))


def test_linear_ref_scaling_identity():
    # the dequantized W' times x/s equals the (quantized) layer applied to x
    g = 64
    w = _random_wp(16, 256, 81)
    x = S.activations(4, 256, 82)
    s = O.scale_candidate(O.calib_stats(S.activations(8, 256, 83, np.array([7, 99]), 20.0)), 0.5)
    inv = O.fp16_rn(1.0 / s.astype(np.float64))
    qw, sc, qz, _ = O.pack_int4(w, s, g)
    y1 = O.linear_ref(x, qw, sc, qz, inv, 256, g)
    x_pre = (x.astype(np.float64) * inv.astype(np.float64)[None, :])
    y2 = x_pre @ O.dequantized_weight(qw, sc, qz, 256, g).T
    assert np.allclose(y1, y2, rtol=0, atol=1e-12)
    # and approximates the float layer W x within the quantization error scale
    yf = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.sqrt(np.mean((y1 - yf) ** 2)) < 0.2 * np.sqrt(np.mean(yf ** 2))


def test_check_linear_floor():
    yr = np.array([[1.0, -2.0, 1e-6, 0.5]])
    ok, worst, raw = O.check_linear(yr.astype(np.float16), yr)
    assert ok and worst < 0.2
    bad = yr.copy()
    bad[0, 1] *= 1.01
    ok, worst, raw = O.check_linear(bad.astype(np.float16), yr)
    assert not ok


# ---------------------------------------------------------------- shared scale, folded 1/s


def test_fold_inv_scale_special_cases():
    r = _rng(90)
    v = (r.standard_normal(512) * 3.0).astype(np.float16)
    assert np.array_equal(O.fold_inv_scale(v, np.ones(512, np.float16)).view(np.uint16), v.view(np.uint16))
    for e in (-14, -3, 0, 2, 5):
        s = np.full(512, 2.0 ** e, np.float16)
        want = O.fp16_rn(v.astype(np.float64) * 2.0 ** -e)     # exact scaling, then one rounding
        assert np.array_equal(O.fold_inv_scale(v, s).view(np.uint16), want.view(np.uint16))


def test_fold_inv_scale_exact_quotient():
    r = _rng(91)
    v = (r.standard_normal(3000) * 10.0 ** r.integers(-4, 3, 3000)).astype(np.float16)
    s = O.scale_candidate(np.abs(r.standard_normal(3000)) * 10.0 ** r.integers(-3, 3, 3000), 0.7)
    got = O.fold_inv_scale(v, s)
    for a, b, h in zip(v, s, got):
        want = X.f16_round_exact(X.frac_of_f16(a) / X.frac_of_f16(b))
        assert float(h) == want or (np.isinf(want) and np.isinf(float(h))), (a, b, float(h), want)


def test_fold_inv_scale_rows():
    r = _rng(97)
    w = (r.standard_normal((40, 24)) * 10.0 ** r.integers(-3, 2, (40, 24))).astype(np.float16)
    s = O.scale_candidate(np.abs(r.standard_normal(40)) * 10.0 ** r.integers(-2, 3, 40), 0.6)
    got = O.fold_inv_scale_rows(w, s)
    # identity and exact power-of-two scaling
    assert np.array_equal(O.fold_inv_scale_rows(w, np.ones(40, np.float16)).view(np.uint16), w.view(np.uint16))
    p2 = np.full(40, 0.25, np.float16)
    assert np.array_equal(O.fold_inv_scale_rows(w, p2).view(np.uint16),
                          O.fp16_rn(w.astype(np.float64) * 4.0).view(np.uint16))
    # every element the exact rational quotient rounded once
    for j in range(0, 40, 7):
        for c in range(24):
            want = X.f16_round_exact(X.frac_of_f16(w[j, c]) / X.frac_of_f16(s[j]))
            assert float(got[j, c]) == want or (np.isinf(want) and np.isinf(float(got[j, c])))
    # row j is the per-channel fold of that row with s_j repeated
    for j in range(40):
        assert np.array_equal(got[j].view(np.uint16),
                              O.fold_inv_scale(w[j], np.full(24, s[j], np.float16)).view(np.uint16))


def test_joint_loss_is_sum_of_stacked_projections():
    # q, k, v read one input: with one s for all three, the loss of their
    # stacked weights is the sum of their own losses, for every alpha
    k, m, g = 64, 5, 32
    ws = [S.weights(n, k, 0.02, 92 + n) for n in (6, 3, 2)]
    x = S.activations(m, k, 95, S.outlier_channels(k, 0.05, 96), 20.0)
    a = O.calib_stats(x)
    for alpha in O.alpha_grid(20)[::4]:
        s16 = O.scale_candidate(a, alpha)
        parts = sum(O.search_loss(w, x, s16, g) for w in ws)
        joint = O.search_loss(np.concatenate(ws), x, s16, g)
        assert abs(joint - parts) <= 1e-12 * abs(parts)


# ---------------------------------------------------------------- other weight widths (3, 8 bits)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g", [32, 128])
def test_codes_brute_force_all_levels_wbit(w_bit, g):
    max_int = (1 << w_bit) - 1
    wp = _random_wp(6, 2 * g, 200 + g + w_bit)
    wp[0, :g] = np.abs(wp[0, :g]) + np.float16(0.5)
    wp[1, g:] = np.float16(-0.75)
    wp[2, :g] = (wp[2, :g].astype(np.float64) * 1e-3).astype(np.float16)
    wp[3, g:] = (wp[3, g:].astype(np.float64) * 3000).astype(np.float16)
    d16, z, bad = O.group_params(wp, g, max_int)
    q = O.quantize_codes(wp, d16, z, g, bad, max_int)
    assert not bad.any() and q.min() >= 0 and q.max() <= max_int
    for r in range(wp.shape[0]):
        steps, zeros, codes = X.exact_group_quant(wp[r], g, max_int)
        assert list(d16[r].astype(np.float64)) == steps, r
        assert list(z[r]) == zeros, r
        assert list(q[r]) == codes, r


@pytest.mark.parametrize("w_bit", [3, 8])
def test_known_answer_random_groups_wbit(w_bit):
    max_int = (1 << w_bit) - 1
    g, n, ng = 64, 6, 3
    r = _rng(40 + w_bit)
    # at most 3 significant bits, so (q - z) * d0 (|q - z| <= 255) is exact in fp16
    d0 = (2.0 ** r.integers(-12, -6, (n, ng)) * (1 + r.integers(0, 4, (n, ng)) / 4)).astype(np.float16)
    z0 = r.integers(0, max_int + 1, (n, ng))
    q0 = r.integers(0, max_int + 1, (n, ng, g))
    q0[:, :, 0] = 0
    q0[:, :, 1] = max_int
    wp = ((q0 - z0[:, :, None]) * d0.astype(np.float64)[:, :, None]).reshape(n, ng * g).astype(np.float16)
    d16, z, bad = O.group_params(wp, g, max_int)
    q = O.quantize_codes(wp, d16, z, g, bad, max_int)
    assert np.array_equal(d16, d0) and np.array_equal(z, z0)
    assert np.array_equal(q.reshape(n, ng, g), q0)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g", [32, 128])
def test_pack_wbit_roundtrip(w_bit, g):
    max_int = (1 << w_bit) - 1
    w = _random_wp(5, 3 * g if g == 128 else 9 * g, 50 + w_bit)
    k = w.shape[1]
    qw, sc, qz, nbad = O.pack_weights(w, None, g, w_bit)
    assert nbad == 0
    _, q2, z2, d2, _, _ = O.fake_quantize(w, None, g, max_int)
    q, z = O.unpack_weights(qw, qz, k, g, w_bit)
    assert np.array_equal(q, q2) and np.array_equal(z, z2) and np.array_equal(sc, d2)
    # the bit positions, checked by hand on row 1
    row = [int(v) for v in qw[1]]
    if w_bit == 8:
        assert qw.shape == (5, k // 4) and qz.shape == (5, -(-(k // g) // 4))
        assert (row[2] >> 8) & 0xFF == q2[1, 9]                  # k = 9: word 2, byte 1
    else:
        assert qw.shape == (5, 3 * k // 32) and qz.shape == (5, -(-(k // g) // 8))
        big = row[3] | (row[4] << 32) | (row[5] << 64)          # codes 32..63
        for kk in (0, 10, 21, 31):                              # 10 and 21 straddle words
            assert (big >> (3 * kk)) & 7 == q2[1, 32 + kk]
        assert (row[0] >> 30) | ((row[1] & 1) << 2) == q2[1, 10]


@pytest.mark.parametrize("w_bit", [3, 8])
def test_alpha0_is_plain_rtn_wbit(w_bit):
    w = _random_wp(3, 64, 61 + w_bit)
    x = S.activations(4, 64, 62, np.array([1, 9]), 20.0)
    a = O.calib_stats(x)
    best, s16, inv, losses = O.search_scale(w, x, a, g=32, n_grid=4, w_bit=w_bit)
    want = _textbook_rtn_error(w, x, 32, (1 << w_bit) - 1)
    assert abs(losses[0] - float(want)) <= 1e-12 * float(want)
    # fewer bits, larger error at the same s
    l3 = O.search_loss(w, x, np.ones(64, np.float16), 32, 7)
    l4 = O.search_loss(w, x, np.ones(64, np.float16), 32, 15)
    l8 = O.search_loss(w, x, np.ones(64, np.float16), 32, 255)
    assert l3 > l4 > l8


def test_bf16_decode():
    # bf16 is the upper 16 bits of an IEEE binary32: values fixed by the format
    bits = np.array([0x3F80, 0xC020, 0x4049, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x0080, 0x7F7F],
                    np.uint16)
    want = [1.0, -2.5, 3.140625, 0.0, -0.0, np.inf, -np.inf, 2.0 ** -133, 2.0 ** -126,
            (2 - 2.0 ** -7) * 2.0 ** 127]
    got = O.bf16_to_f64(bits)
    for g_, w_ in zip(got, want):
        assert g_ == w_ and np.signbit(g_) == np.signbit(w_)
    assert np.isnan(O.bf16_to_f64(np.array([0x7FC0], np.uint16))[0])
    with pytest.raises(TypeError):
        O.exact_f64(np.array([1, 2], np.int32))


def test_linear_ref_bf16_exact_small():
    # bf16 activations (float64 values) against a rational sum over the unpacked bits
    g = 32
    w = _random_wp(3, 64, 91)
    xb = S.activations_bf16(2, 64, 92, np.array([3]), 40.0)
    x = O.bf16_to_f64(xb)
    s = O.scale_candidate(O.calib_stats(S.activations(8, 64, 93, np.array([5]), 20.0)), 0.4)
    inv = O.fp16_rn(1.0 / s.astype(np.float64))
    qw, sc, qz, _ = O.pack_int4(w, s, g)
    y = O.linear_ref(x, qw, sc, qz, inv, 64, g)
    for t in range(2):
        for n in range(3):
            acc = Fraction(0)
            for c in range(64):
                code = (int(qw[n, c // 8]) >> (4 * (c % 8))) & 0xF
                j = c // g
                zero = (int(qz[n, j // 8]) >> (4 * (j % 8))) & 0xF
                acc += Fraction(float(x[t, c])) * Fraction(float(inv[c])) * (code - zero) * Fraction(float(sc[n, j]))
            assert abs(y[t, n] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc)))
    # the generator's draws are those of the fp16 generator, rounded to bf16
    xh = S.activations(2, 64, 92, np.array([3]), 40.0).astype(np.float64)
    assert np.all(np.abs(x - xh) <= 2.0 ** -8 * np.abs(xh) + 2.0 ** -10 * np.abs(xh) + 1e-30)


def test_salient_channels_brute_force():
    r = np.random.Generator(np.random.PCG64(2501))
    for trial in range(200):
        k = int(r.integers(1, 8))
        a = r.integers(0, 4, size=k).astype(np.float64)     # many ties
        if trial % 5 == 0:
            a[int(r.integers(0, k))] = np.nan
        if trial % 7 == 0:
            a[int(r.integers(0, k))] = np.inf
        rank = np.where(np.isnan(a), np.inf, a)
        for count in range(k + 1):
            sel = O.salient_channels(a, count)
            assert len(sel) == count and np.all(np.diff(sel) > 0)
            chosen = np.zeros(k, bool)
            chosen[sel] = True
            for i in range(k):
                for j in range(k):
                    if chosen[i] and not chosen[j]:
                        # i outranks j: NaN first, then larger a, then lower index
                        ki = (np.isnan(a[i]), rank[i], -i)
                        kj = (np.isnan(a[j]), rank[j], -j)
                        assert ki > kj, (a, count, sel)


def test_salient_count():
    assert O.salient_count(4096, 0.01) == 41
    assert O.salient_count(14336, 0.01) == 143
    assert O.salient_count(100, 0.005) == 1          # 0.5 rounds up
    assert O.salient_count(10, 0.0) == 0 and O.salient_count(10, 2.0) == 10


def test_mixed_loss_two_ways():
    # protecting channels removes their error columns, which is the search loss
    # at s = 1 on activations whose protected channels are zero
    g = 32
    w = S.weights(24, 256, 0.02, 2511)
    ch = S.outlier_channels(256, 0.03, 2512)
    x = S.activations(40, 256, 2513, ch, 30.0)
    a = O.calib_stats(x)
    idx = O.salient_channels(a, 5)
    assert set(idx.tolist()) <= set(ch.tolist())       # the outlier channels rank first
    xm = x.copy()
    xm[:, idx] = 0
    lm = O.mixed_loss(w, x, idx, g)
    l0 = O.search_loss(w, xm, np.ones(256, np.float16), g)
    assert abs(lm - l0) <= 1e-12 * l0
    # and protecting the outlier channels beats plain RTN on this input
    assert lm < 0.5 * O.search_loss(w, x, np.ones(256, np.float16), g)


def test_mixed_extremes():
    g = 64
    w = S.weights(8, 128, 0.02, 2521)
    x = S.activations(16, 128, 2522)
    none = np.zeros(0, np.int32)
    assert O.mixed_loss(w, x, none, g) == O.search_loss(w, x, np.ones(128, np.float16), g)
    assert O.mixed_loss(w, x, np.arange(128, dtype=np.int32), g) == 0.0
    wm = O.mixed_weight(w, np.array([3, 77], np.int32), g)
    assert np.array_equal(wm[:, [3, 77]], w[:, [3, 77]].astype(np.float64))


def test_linear_mixed_ref_exact_small():
    g = 32
    w = _random_wp(3, 64, 2531)
    x = S.activations(2, 64, 2532, np.array([9]), 30.0)
    idx = np.array([9, 40], np.int32)
    qw, sc, qz, _ = O.pack_int4(w, None, g)
    y = O.linear_mixed_ref(x, qw, sc, qz, w, idx, 64, g)
    for t in range(2):
        for n in range(3):
            acc = Fraction(0)
            for c in range(64):
                if c in (9, 40):
                    wv = Fraction(float(w[n, c]))
                else:
                    code = (int(qw[n, c // 8]) >> (4 * (c % 8))) & 0xF
                    j = c // g
                    zero = (int(qz[n, j // 8]) >> (4 * (j % 8))) & 0xF
                    wv = (code - zero) * Fraction(float(sc[n, j]))
                acc += Fraction(float(x[t, c])) * wv
            assert abs(y[t, n] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc)))
