"""GPU parity for 3- and 8-bit weights (awq_search_scale_wbit, awq_pack_wbit,
awq_linear_wbit) against the CPU oracle's max_int = 2^w_bit - 1 rule:
bit-exact chosen alpha, s16, inv_s16, packed codes, zero points and fp16
scales; linear outputs within the floored relative tolerance 5e-3 against
float64.  w_bit = 4 through the same entries equals the 4-bit entries bit for
bit."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O
from tests import search_bound as SB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def P():
    import weight_only_int4_awq_amd as P
    P.load()
    assert torch.cuda.is_available()
    return P


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def u16(t):
    return t.cpu().numpy().view(np.uint16)


def _check_pack(P, w, s16, g, w_bit, rows=None):
    qw, sc, qz, bad = P.awq_pack_wbit(dev(w), None if s16 is None else dev(s16), g=g,
                                      w_bit=w_bit)
    torch.cuda.synchronize()
    wr = w if rows is None else w[rows]
    oqw, osc, oqz, obad = O.pack_weights(wr, s16, g, w_bit)
    hq, hs, hz = u32(qw), u16(sc), u32(qz)
    if rows is not None:
        hq, hs, hz = hq[rows], hs[rows], hz[rows]
    assert np.array_equal(hq, oqw)
    assert np.array_equal(hs, osc.view(np.uint16))
    assert np.array_equal(hz, oqz)
    if rows is None:
        assert int(bad.item()) == obad
    return qw, sc, qz


# ----------------------------------------------------------------- pack


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("n,k", [(1, 128), (33, 384), (7, 2048 + 384), (300, 4096)])
def test_pack_wbit_bit_exact(P, w_bit, g, n, k):
    if k % g:
        pytest.skip("k must be a multiple of g")
    w = S.weights(n, k, 0.02, 1077 + n + k)
    _check_pack(P, w, None, g, w_bit)
    x = S.activations(64, k, 1078, S.outlier_channels(k, 0.01, 1079), 20.0)
    s16 = O.scale_candidate(O.calib_stats(x), 0.45)
    _check_pack(P, w, s16, g, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
def test_pack_wbit_ties_and_edge_groups(P, w_bit):
    g = 32
    max_int = (1 << w_bit) - 1
    d = 2.0 ** -7 if w_bit == 3 else 2.0 ** -10
    lo = -(max_int // 2)
    w = S.weights(5, 4 * g, 0.02, 1091)
    # a group of range max_int * d holding exact half-steps: every rounding tie
    w[0, :g] = np.float16(0)
    w[0, 0], w[0, 1] = np.float16(lo * d), np.float16((lo + max_int) * d)
    for i, h in enumerate((0.5, 1.5, 2.5, -0.5, -1.5, -2.5, lo + 0.5, lo + max_int - 0.5)):
        w[0, 2 + i] = np.float16(h * d)
    w[1, :g] = np.float16(0.3)                                  # constant group (range floor)
    w[1, g:2 * g] = np.abs(w[1, g:2 * g]) + np.float16(1.0)       # no zero in range
    w[2, :g] = (w[2, :g].astype(np.float64) * 1e-3).astype(np.float16)
    w[3, :g] = (w[3, :g].astype(np.float64) * 2000).astype(np.float16)
    w[4, :g] = np.abs(w[4, :g])                                   # zero point at 0
    w[4, g:2 * g] = -np.abs(w[4, g:2 * g])                        # zero point at max_int
    _check_pack(P, w, None, g, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
def test_pack_wbit_nonfinite_groups(P, w_bit):
    g = 64
    w = S.weights(3, 256, 0.02, 1095)
    w[1, 70] = np.float16(np.nan)
    w[2, 200] = np.float16(np.inf)
    s16 = np.ones(256, np.float16)
    s16[10] = np.float16(60000.0)
    w[0, 10] = np.float16(3.0)
    _check_pack(P, w, s16, g, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_pack_wbit_full_size_sampled_rows(P, w_bit, name, n, k):
    w, x_cal, _, _ = S.config_layer(2, name, n, k, 128, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    rows = np.sort(np.random.Generator(np.random.PCG64(n + k + w_bit)).choice(n, 128, replace=False))
    _check_pack(P, w, s16, 128, w_bit, rows=rows)


def test_pack_wbit_4_is_pack_int4(P):
    w = S.weights(40, 640, 0.02, 1101)
    wd = dev(w)
    a = P.awq_pack_wbit(wd, None, g=64, w_bit=4)
    b = P.awq_pack_int4(wd, None, g=64)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ----------------------------------------------------------------- search


def _check_search(P, w, x, g, n_grid, w_bit):
    a_dev = P.awq_calib_stats(dev(x))
    best, s16, inv, losses = P.awq_search_scale_wbit(dev(w), dev(x), a_dev, g=g, n_grid=n_grid,
                                                     w_bit=w_bit)
    torch.cuda.synchronize()
    a = O.calib_stats(x)
    ob, os16, oinv, olosses = O.search_scale(w, x, a, g=g, n_grid=n_grid, w_bit=w_bit)
    # the bound of the 4-bit search (the same kernel; tests/search_bound.py)
    dnorm = SB.loss_bounds(w, x, a, g, n_grid, w_bit)
    worst = SB.check_losses(losses.cpu().numpy(), olosses, dnorm)
    b, second, gap, margin = SB.gap_report(olosses, dnorm)
    print(f"search gap [w_bit {w_bit} {w.shape} m={x.shape[0]} g={g}]: best {ob} second {second} "
          f"gap {gap:.3e} margin {margin:.3g} max rel loss err {worst:.2e}")
    assert int(best.item()) == ob, (int(best.item()), ob, gap, margin)
    assert np.array_equal(u16(s16), os16.view(np.uint16))
    assert np.array_equal(u16(inv), oinv.view(np.uint16))
    return ob


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("n,k,m,g", [(40, 256, 20, 64), (70, 384, 130, 128), (33, 96, 5, 32),
                                      (64, 512, 600, 128)])
def test_search_wbit_small(P, w_bit, n, k, m, g):
    w = S.weights(n, k, 0.02, 1300 + n)
    x = S.activations(m, k, 1301 + m, S.outlier_channels(k, 0.02, 1302), 20.0)
    _check_search(P, w, x, g, 20, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
def test_search_wbit_full_k_sampled_rows(P, w_bit):
    # the Llama-3-8B down projection's full K with 512 calibration tokens on 64 rows
    n, k = 4096, 14336
    w, x_cal, _, _ = S.config_layer(3, "down", n, k, 512, 0, 0.02, 0.01, 20.0)
    rows = np.sort(np.random.Generator(np.random.PCG64(n + w_bit)).choice(n, 64, replace=False))
    _check_search(P, np.ascontiguousarray(w[rows]), x_cal, 128, 20, w_bit)


def test_search_wbit_4_is_search_scale(P):
    w = S.weights(64, 512, 0.02, 1311)
    x = S.activations(100, 512, 1312, S.outlier_channels(512, 0.02, 1313), 20.0)
    wd, xd = dev(w), dev(x)
    a = P.awq_calib_stats(xd)
    r1 = P.awq_search_scale_wbit(wd, xd, a, g=128, w_bit=4)
    r2 = P.awq_search_scale(wd, xd, a, g=128)
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


def test_search_wbit_fewer_bits_lose_more(P):
    # the quantization error at the chosen alpha shrinks with the code width
    w = S.weights(96, 512, 0.02, 1321)
    x = S.activations(64, 512, 1322, S.outlier_channels(512, 0.02, 1323), 20.0)
    wd, xd = dev(w), dev(x)
    a = P.awq_calib_stats(xd)
    best = {}
    for wb in (3, 4, 8):
        b, _, _, losses = P.awq_search_scale_wbit(wd, xd, a, w_bit=wb)
        torch.cuda.synchronize()
        best[wb] = float(losses.cpu().numpy()[int(b.item())])
    assert best[3] > best[4] > best[8] > 0


# ----------------------------------------------------------------- linear


def _check_linear(P, w, x, s16, g, w_bit, cols=None):
    """GPU linear on the oracle's pack (uploaded) against the oracle."""
    inv = None if s16 is None else O.fp16_rn(1.0 / s16.astype(np.float64))
    hq, hs, hz, _ = O.pack_weights(w, s16, g, w_bit)
    qw, sc, qz = dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32))
    y = P.awq_linear_wbit(dev(x), qw, sc, qz, None if inv is None else dev(inv), g=g, w_bit=w_bit)
    torch.cuda.synchronize()
    k = w.shape[1]
    yh = y.cpu().numpy().astype(np.float16)
    if cols is None:
        yr = O.linear_ref(x, hq, hs, hz, inv, k, g, w_bit)
        ok, worst, raw = O.check_linear(yh, yr)
    else:
        yr = O.linear_ref_rows(x, hq, hs, hz, inv, k, g, cols, w_bit)
        ok, worst, raw = O.check_linear(yh[:, cols], yr)
    assert ok, (worst, raw)
    return worst


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 300])
def test_linear_wbit_small(P, w_bit, g, m):
    n, k = 50, 640
    w = S.weights(n, k, 0.02, 1400 + m)
    x = S.activations(m, k, 1401 + m, S.outlier_channels(k, 0.01, 1402), 20.0)
    xc = S.activations(64, k, 1403, S.outlier_channels(k, 0.01, 1402), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.4)
    _check_linear(P, w, x, s16, g, w_bit)
    _check_linear(P, w, x, None, g, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("n,k", [(16, 64), (257, 1152), (129, 4096)])
def test_linear_wbit_ragged(P, w_bit, n, k):
    for m in (1, 8, 40):
        w = S.weights(n, k, 0.02, 1410 + n)
        x = S.activations(m, k, 1411 + m)
        _check_linear(P, w, x, None, 64 if k % 128 else 128, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_linear_wbit_decode_full_size(P, w_bit, name, n, k):
    w, x_cal, x_run, _ = S.config_layer(2, name, n, k, 128, 1, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    _check_linear(P, w, x_run, s16, 128, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("name,n,k", [("gate", 14336, 4096), ("down", 4096, 14336)])
def test_linear_wbit_32_tokens_full_size_sampled(P, w_bit, name, n, k):
    # 17-32 tokens run the tiled GEMM with 64-row tiles, split along K (two
    # work-groups per CU of K slices for down, K >= 8192): full Llama-3-8B
    # gate and down shapes at 24 and 32 tokens on sampled columns
    w, x_cal, _, _ = S.config_layer(2, name, n, k, 128, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    inv = O.fp16_rn(1.0 / s16.astype(np.float64))
    hq, hs, hz, _ = O.pack_weights(w, s16, 128, w_bit)
    del w
    qw, sc, qz = dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32))
    rng = np.random.Generator(np.random.PCG64(1480 + n + w_bit))
    cols = np.unique(np.concatenate([rng.choice(n, 128, replace=False), np.arange(n - 8, n)]))
    ch = S.outlier_channels(k, 0.01, S.seed_of(2, 0, S.SLOTS[S.INPUT_OF[name]], 3))
    for m in (24, 32):
        x = S.activations(m, k, 1481 + m, ch, 20.0)
        y = P.awq_linear_wbit(dev(x), qw, sc, qz, dev(inv), g=128, w_bit=w_bit)
        torch.cuda.synchronize()
        yr = O.linear_ref_rows(x, hq, hs, hz, inv, k, 128, cols, w_bit)
        ok, worst, raw = O.check_linear(y.cpu().numpy()[:, cols], yr)
        assert ok, (m, worst, raw)


@pytest.mark.parametrize("w_bit", [3, 8])
def test_linear_wbit_prefill_full_size_sampled(P, w_bit):
    n, k = 14336, 4096
    w, x_cal, x_run, _ = S.config_layer(3, "gate", n, k, 512, 2048, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    cols = np.sort(np.random.Generator(np.random.PCG64(n + w_bit)).choice(n, 64, replace=False))
    _check_linear(P, w, x_run, s16, 128, w_bit, cols=cols)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g,k", [(64, 1856), (32, 960), (128, 3712), (32, 14336)])
def test_linear_wbit_gemm_windows(P, w_bit, g, k):
    # the GEMM restages scales every 28 groups: K ranges that end in a
    # one-step window, a short window and 16 windows; tiles of 64 and 256 rows
    # with ragged m and n
    n = 200
    w = S.weights(n, k, 0.02, 1450 + k)
    xc = S.activations(64, k, 1451, S.outlier_channels(k, 0.01, 1452), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.5)
    for m in (33, 129, 300):
        x = S.activations(m, k, 1453 + m, S.outlier_channels(k, 0.01, 1452), 20.0)
        _check_linear(P, w, x, s16, g, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
def test_linear_wbit_decode_long_k(P, w_bit):
    # k = 28672 (the Llama-3-70B down projection's K): one token's x_tilde and
    # scale table take more than 64 KiB of LDS, two tokens more than 128 KiB,
    # three do not fit and take the unstaged kernel
    n, k = 257, 28672
    w = S.weights(n, k, 0.015, 1460)
    xc = S.activations(32, k, 1461, S.outlier_channels(k, 0.005, 1462), 30.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.5)
    for m in (1, 2, 3):
        x = S.activations(m, k, 1463 + m, S.outlier_channels(k, 0.005, 1462), 30.0)
        _check_linear(P, w, x, s16, 128, w_bit)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("g", [64, 128])
def test_linear_wbit_decode_many_blocks(P, w_bit, g):
    # 1101 column blocks (the last one ragged): work-groups of the staged
    # decode kernel own 3 blocks, some of the last ones fewer
    n, k = 16 * 1100 + 5, 1024
    w = S.weights(n, k, 0.02, 1470)
    cols = np.sort(np.random.Generator(np.random.PCG64(1471)).choice(n, 300, replace=False))
    cols[-1] = n - 1
    for m in (1, 3):
        x = S.activations(m, k, 1472 + m, S.outlier_channels(k, 0.01, 1473), 20.0)
        _check_linear(P, w, x, None, g, w_bit, cols=np.unique(cols))


def test_linear_wbit_4_is_linear_w4a16(P):
    w = S.weights(96, 1024, 0.02, 1431)
    qw, sc, qz, _ = P.awq_pack_int4(dev(w), None, g=128)
    for m in (1, 8, 40):
        x = dev(S.activations(m, 1024, 1432 + m))
        a = P.awq_linear_wbit(x, qw, sc, qz, None, g=128, w_bit=4)
        b = P.awq_linear_w4a16(x, qw, sc, qz, None, g=128)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_linear_wbit_deterministic(P):
    w = S.weights(300, 2048, 0.02, 1441)
    inv = dev(np.full(2048, 0.5, np.float16))
    for wb in (3, 8):
        qw, sc, qz, _ = P.awq_pack_wbit(dev(w), None, g=128, w_bit=wb)
        for m in (20, 300):
            x = dev(S.activations(m, 2048, 1442))
            a = P.awq_linear_wbit(x, qw, sc, qz, inv, g=128, w_bit=wb)
            b = P.awq_linear_wbit(x, qw, sc, qz, inv, g=128, w_bit=wb)
            torch.cuda.synchronize()
            assert torch.equal(a, b)
