"""GPU parity: every entry point of the C ABI against the CPU oracle on the same
seeded inputs.  Bit-exact for the statistic, the packed nibbles, zero points,
fp16 scales, s16, inv_s16 and the chosen alpha; the linear outputs within the
floored relative tolerance 5e-3 against float64.

Small shapes span several tiles and a ragged tail; full Llama-shaped sizes are
checked on sampled rows / columns the oracle computes one by one."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O

from tests import search_bound as SB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def P():
    import weight_only_int4_awq_amd as P
    P.load()
    assert torch.cuda.is_available()
    return P


DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host16(t):
    return t.cpu().numpy().astype(np.float16)


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


# ----------------------------------------------------------------- calib stats


@pytest.mark.parametrize("m,k", [(1, 8), (37, 264), (128, 4096), (512, 14336), (8192, 64)])
def test_calib_stats_bit_exact(P, m, k):
    x = S.activations(m, k, 1000 + m, S.outlier_channels(k, 0.01, 7), 20.0)
    got = P.awq_calib_stats(dev(x)).cpu().numpy()
    want = O.calib_stats(x)
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


def test_calib_stats_nonfinite(P):
    x = S.activations(16, 64, 5)
    x[3, 5] = np.float16(np.inf)
    x[4, 9] = np.float16(-np.inf)
    x[2, 9] = np.float16(np.nan)
    got = P.awq_calib_stats(dev(x)).cpu().numpy()
    want = O.calib_stats(x)
    assert np.isinf(got[5]) and np.isnan(got[9]) and np.isnan(want[9])
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])


# ----------------------------------------------------------------- pack


def _check_pack(P, w, s16, g):
    qw, sc, qz, bad = P.awq_pack_int4(dev(w), None if s16 is None else dev(s16), g=g)
    torch.cuda.synchronize()
    oqw, osc, oqz, obad = O.pack_int4(w, s16, g)
    assert np.array_equal(host_u32(qw), oqw)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), osc.view(np.uint16))
    assert np.array_equal(host_u32(qz), oqz)
    assert int(bad.item()) == obad


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("n,k", [(1, 128), (33, 384), (7, 2048 + 384), (300, 4096)])
def test_pack_bit_exact(P, g, n, k):
    if k % g:
        pytest.skip("k must be a multiple of g")
    w = S.weights(n, k, 0.02, 77 + n + k)
    _check_pack(P, w, None, g)
    x = S.activations(64, k, 78, S.outlier_channels(k, 0.01, 79), 20.0)
    s16 = O.scale_candidate(O.calib_stats(x), 0.45)
    _check_pack(P, w, s16, g)


def test_pack_ties_and_edge_groups(P):
    g = 32
    d = 2.0 ** -7
    w = S.weights(4, 4 * g, 0.02, 91)
    # exact half-step values in a group of range 15 d: every rounding tie
    w[0, :g] = np.float16(0)
    w[0, 0], w[0, 1] = np.float16(-7 * d), np.float16(8 * d)
    for i, h in enumerate((0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, 7.5, -6.5)):
        w[0, 2 + i] = np.float16(h * d)
    w[1, :g] = np.float16(0.3)                      # constant group (range floor)
    w[1, g:2 * g] = np.abs(w[1, g:2 * g]) + np.float16(1.0)   # no zero in range
    w[2, :g] = (w[2, :g].astype(np.float64) * 1e-3).astype(np.float16)   # subnormal-ish
    w[3, :g] = (w[3, :g].astype(np.float64) * 2000).astype(np.float16)   # large values
    _check_pack(P, w, None, g)


def test_pack_nonfinite_groups(P):
    g = 64
    w = S.weights(3, 256, 0.02, 95)
    w[1, 70] = np.float16(np.nan)
    w[2, 200] = np.float16(np.inf)
    s16 = np.ones(256, np.float16)
    s16[10] = np.float16(60000.0)
    w[0, 10] = np.float16(3.0)
    _check_pack(P, w, s16, g)


@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_pack_full_size_sampled_rows(P, name, n, k):
    w, x_cal, _, _ = S.config_layer(2, name, n, k, 128, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    qw, sc, qz, bad = P.awq_pack_int4(dev(w), dev(s16), g=128)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(n + k)).choice(n, 256, replace=False))
    oqw, osc, oqz, obad = O.pack_int4(w[rows], s16, 128)
    assert np.array_equal(host_u32(qw)[rows], oqw)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16)[rows], osc.view(np.uint16))
    assert np.array_equal(host_u32(qz)[rows], oqz)
    assert int(bad.item()) == 0


# ----------------------------------------------------------------- search


def _check_search(P, w, x, g, n_grid, expect_best=None, label=None):
    """GPU search against the oracle: alpha index, s16 and inv_s16 bit for bit,
    every loss within the bound derived from the kernel's arithmetic
    (tests/search_bound.py).  Prints the oracle's best-vs-second gap and its
    margin over the two losses' bounds (margin > 1: the index cannot flip)."""
    a_dev = P.awq_calib_stats(dev(x))
    best, s16, inv, losses = P.awq_search_scale(dev(w), dev(x), a_dev, g=g, n_grid=n_grid)
    torch.cuda.synchronize()
    a = O.calib_stats(x)
    ob, os16, oinv, olosses = O.search_scale(w, x, a, g=g, n_grid=n_grid)
    dnorm = SB.loss_bounds(w, x, a, g, n_grid)
    worst = SB.check_losses(losses.cpu().numpy(), olosses, dnorm)
    b, second, gap, margin = SB.gap_report(olosses, dnorm)
    print(f"search gap [{label or (w.shape, x.shape[0], g)}]: best {ob} second {second} "
          f"gap {gap:.3e} margin {margin:.3g} max rel loss err {worst:.2e}")
    assert int(best.item()) == ob, (int(best.item()), ob, gap, margin)
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), os16.view(np.uint16))
    assert np.array_equal(inv.cpu().numpy().view(np.uint16), oinv.view(np.uint16))
    if expect_best is not None:
        assert ob == expect_best
    return ob, gap


@pytest.mark.parametrize("n,k,m,g", [(40, 256, 20, 64), (70, 384, 130, 128), (33, 96, 5, 32),
                                      (64, 512, 600, 128), (1, 128, 1, 128)])
def test_search_small(P, n, k, m, g):
    w = S.weights(n, k, 0.02, 300 + n)
    x = S.activations(m, k, 301 + m, S.outlier_channels(k, 0.02, 302), 20.0)
    _check_search(P, w, x, g, 20)


def test_search_tie_break_constant_activations(P):
    w = S.weights(48, 256, 0.02, 311)
    x = np.where(np.random.Generator(np.random.PCG64(312)).random((16, 256)) < 0.5, -1.0,
                 1.0).astype(np.float16)
    _check_search(P, w, x, 128, 20, expect_best=0)


def test_search_nonfinite_alpha(P):
    # a huge activation column makes large alphas overflow W * s: those get an infinite loss
    w = S.weights(32, 128, 0.5, 321)
    x = S.activations(8, 128, 322)
    x[:, 3] = np.float16(60000.0)
    w[0, 3] = np.float16(2.0)      # 2 * 60000^0.95 overflows fp16
    ob, gap = _check_search(P, w, x, 128, 20)
    a = O.calib_stats(x)
    assert not np.isfinite(O.search_loss(w, x, O.scale_candidate(a, 0.95), 128))


@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_search_full_k_sampled_rows(P, name, n, k):
    # full K and the calibration set of the Llama-3-8B prefill workload (512 tokens) on 96
    # sampled rows: the loss is a sum over rows, so this is the same search restricted to them
    w, x_cal, _, _ = S.config_layer(3, name, n, k, 512, 0, 0.02, 0.01, 20.0)
    rows = np.sort(np.random.Generator(np.random.PCG64(n)).choice(n, 96, replace=False))
    _check_search(P, np.ascontiguousarray(w[rows]), x_cal, 128, 20)


def test_search_rows_additive_full_size(P):
    # the full 4096 x 4096 search (128 tokens) equals the sum of its row-block searches
    w, x_cal, _, _ = S.config_layer(1, "q", 4096, 4096, 128, 0, 0.02, 0.01, 20.0)
    wd, xd = dev(w), dev(x_cal)
    a = P.awq_calib_stats(xd)
    best, s16, inv, losses = P.awq_search_scale(wd, xd, a)
    parts = [P.awq_search_scale(wd[i:i + 1024].contiguous(), xd, a)[3] for i in range(0, 4096, 1024)]
    torch.cuda.synchronize()
    tot = sum(p.cpu().numpy() for p in parts)
    full = losses.cpu().numpy()
    assert np.max(np.abs(tot - full) / full) < 1e-12
    # and the 128 sampled rows agree with the oracle
    rows = np.arange(0, 4096, 32)
    _check_search(P, np.ascontiguousarray(w[rows]), x_cal, 128, 20)


def test_search_deterministic(P):
    w = S.weights(256, 1024, 0.02, 331)
    x = S.activations(200, 1024, 332, S.outlier_channels(1024, 0.01, 333), 20.0)
    wd, xd = dev(w), dev(x)
    a = P.awq_calib_stats(xd)
    r1 = P.awq_search_scale(wd, xd, a)
    r2 = P.awq_search_scale(wd, xd, a)
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


# ----------------------------------------------------------------- linear


def oracle_pack(w, s16, g):
    """The oracle's pack of w at s16 (CPU), uploaded: (qweight, scales, qzeros) on
    the device and as host arrays.  Linear tests take their packed weights from
    the oracle, never from the GPU pack."""
    hq, hs, hz, _ = O.pack_int4(w, s16, g)
    return (dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32))), (hq, hs, hz)


def _check_linear(P, w, x, s16, g, cols=None):
    inv = None if s16 is None else O.fp16_rn(1.0 / s16.astype(np.float64))
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, s16, g)
    y = P.awq_linear_w4a16(dev(x), qw, sc, qz, None if inv is None else dev(inv), g=g)
    torch.cuda.synchronize()
    k = w.shape[1]
    yh = host16(y)
    if cols is None:
        yr = O.linear_ref(x, hq, hs, hz, inv, k, g)
        ok, worst, raw = O.check_linear(yh, yr)
    else:
        yr = O.linear_ref_rows(x, hq, hs, hz, inv, k, g, cols)
        ok, worst, raw = O.check_linear(yh[:, cols], yr)
    assert ok, (worst, raw)
    return worst, raw


@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 16, 31, 32, 33, 100, 257])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_linear_small(P, m, g):
    n, k = 50, 640
    w = S.weights(n, k, 0.02, 400 + m)
    x = S.activations(m, k, 401 + m, S.outlier_channels(k, 0.01, 402), 20.0)
    xc = S.activations(64, k, 403, S.outlier_channels(k, 0.01, 402), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.4)
    _check_linear(P, w, x, s16, g)
    _check_linear(P, w, x, None, g)


@pytest.mark.parametrize("n,k", [(16, 64), (257, 1152), (129, 4096)])
def test_linear_ragged(P, n, k):
    for m in (1, 8, 40, 300):
        w = S.weights(n, k, 0.02, 410 + n)
        x = S.activations(m, k, 411 + m)
        _check_linear(P, w, x, None, 64)


@pytest.mark.parametrize("g", [128, 64])
@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_linear_decode_full_size(P, name, n, k, g):
    # every output of the Llama-3-8B-shaped linears at the decode sizes, with
    # group sizes 128 and 64 (the stack's two variants): m = 1 the decode GEMV,
    # 8 the fused skinny kernel (group-major where blocks are shared), 24 and 32
    # the two-chunk group-major kernel for q, k, v and o and the grouped GEMM (64-row
    # tiles, split along K) for gate, up and down
    w, x_cal, _, _ = S.config_layer(2, name, n, k, 128, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    inv = O.fp16_rn(1.0 / s16.astype(np.float64))
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, s16, g)
    del w
    ch = S.outlier_channels(k, 0.01, S.seed_of(2, 0, S.SLOTS.get(S.INPUT_OF[name], 0), 3))
    for m in ((1, 8, 24, 32) if g == 128 else (1, 8, 32)):
        x = S.activations(m, k, S.seed_of(2, 0, S.SLOTS[name], 2) + m, ch, 20.0)
        y = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=g)
        torch.cuda.synchronize()
        yr = O.linear_ref(x, hq, hs, hz, inv, k, g)
        ok, worst, raw = O.check_linear(host16(y), yr)
        assert ok, (m, worst, raw)


@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_linear_prefill_full_size_sampled(P, name, n, k):
    w, x_cal, x_run, _ = S.config_layer(3, name, n, k, 512, 2048, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    cols = np.sort(np.random.Generator(np.random.PCG64(n + 1)).choice(n, 96, replace=False))
    _check_linear(P, w, x_run, s16, 128, cols=cols)


@pytest.mark.parametrize("name,n,k", S.LLAMA3_70B_LINEARS)
def test_linear_70b_shapes_sampled(P, name, n, k):
    w = S.weights(n, k, 0.015, S.seed_of(4, 0, S.SLOTS[name], 0))
    ch = S.outlier_channels(k, 0.005, S.seed_of(4, 0, S.SLOTS[name], 3))
    cols = np.sort(np.random.Generator(np.random.PCG64(n + 2)).choice(n, 256, replace=False))
    for m in (1, 16, 24):
        x = S.activations(m, k, S.seed_of(4, 0, S.SLOTS[name], 2), ch, 30.0)
        _check_linear(P, w, x, None, 128, cols=cols)


def test_linear_deterministic(P):
    w = S.weights(512, 2048, 0.02, 431)
    qw, sc, qz, _ = P.awq_pack_int4(dev(w), None, g=128)
    for m in (1, 8, 32, 300):
        x = dev(S.activations(m, 2048, 432 + m))
        y1 = P.awq_linear_w4a16(x, qw, sc, qz, None, g=128)
        y2 = P.awq_linear_w4a16(x, qw, sc, qz, None, g=128)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)


@pytest.mark.parametrize("n,k,g", [(40, 16384, 32), (24, 28672, 64), (33, 8192, 32), (20, 40960, 128),
                                   (16, 65536, 128)])
def test_linear_decode_wide_k(P, n, k, g):
    # long K with small groups: fewer column blocks per work-group fit the
    # decode kernels' prologue and LDS plans (down to one at 28672 / 64); at
    # K = 40960 with g = 128 the m = 1 activations alone exceed LDS and the
    # staged two-kernel path runs at m = 1; at K = 65536 it runs at every m
    w = S.weights(n, k, 0.02, 440 + n)
    for m in (1, 8, 24):
        x = S.activations(m, k, 441 + n + m, S.outlier_channels(k, 0.01, 442), 20.0)
        _check_linear(P, w, x, None, g)


@pytest.mark.parametrize("n,k,g", [(8261, 256, 64), (40000, 512, 128), (12345, 2048, 32)])
def test_linear_decode_multiblock(P, n, k, g):
    # more column blocks than resident work-groups: several blocks per
    # work-group (up to four), a ragged last block, and (k / g < 8) waves that
    # own no group and only meet the barriers
    w = S.weights(n, k, 0.02, 450 + n)
    x = S.activations(1, k, 451 + n, S.outlier_channels(k, 0.01, 452), 20.0)
    xc = S.activations(64, k, 453, S.outlier_channels(k, 0.01, 452), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.3)
    _check_linear(P, w, x, s16, g)


@pytest.mark.parametrize("n,k,g", [(8261, 256, 64), (12345, 2048, 32), (1024, 8192, 128), (20000, 4096, 64),
                                   (3000, 4096, 128)])
def test_linear_decode_rows_multiblock(P, n, k, g):
    # the decode GEMV with token rows (2 <= m <= 8): several column blocks per
    # work-group (up to four with two 8-wave work-groups per CU, up to eight
    # with one 16-wave work-group: 20000 x 4096 at m = 8), a ragged last
    # block, waves that own no group (k / g below the wave count), and at
    # k = 8192 the activations alone filling most of LDS (one block per
    # work-group)
    w = S.weights(n, k, 0.02, 460 + n)
    xc = S.activations(64, k, 463, S.outlier_channels(k, 0.01, 462), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.3)
    inv = O.fp16_rn(1.0 / s16.astype(np.float64))
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, s16, g)
    for m in (2, 5, 8):
        x = S.activations(m, k, 461 + n + m, S.outlier_channels(k, 0.01, 462), 20.0)
        y = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=g)
        torch.cuda.synchronize()
        ok, worst, raw = O.check_linear(host16(y), O.linear_ref(x, hq, hs, hz, inv, k, g))
        assert ok, (m, worst, raw)


@pytest.mark.parametrize("n,k,g", [(12008, 2048, 64), (16008, 2048, 32), (8008, 4096, 128), (700, 8192, 64)])
def test_linear_skinny_two_chunk_multiblock(P, n, k, g):
    # 17 to 32 tokens on linears of at most 16 MiB of packed weights: the
    # group-major kernel with two token chunks, one work-group per CU, so more
    # than 256 column blocks give several per work-group (three at 12008 x 2048,
    # four at 16008 x 2048, two at g = 128, where more would spill), ragged last
    # blocks, tokens of the second chunk partly past m; at k = 8192 one block per
    # work-group
    w = S.weights(n, k, 0.02, 470 + n)
    xc = S.activations(64, k, 473, S.outlier_channels(k, 0.01, 472), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.3)
    inv = O.fp16_rn(1.0 / s16.astype(np.float64))
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, s16, g)
    for m in (17, 24, 32):
        x = S.activations(m, k, 471 + n + m, S.outlier_channels(k, 0.01, 472), 20.0)
        y = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=g)
        torch.cuda.synchronize()
        ok, worst, raw = O.check_linear(host16(y), O.linear_ref(x, hq, hs, hz, inv, k, g))
        assert ok, (m, worst, raw)


def test_linear_packed_weights_at_4gib(P):
    # the largest packed weights a call takes (n k / 2 just below 4 GiB): the
    # decode kernels' 32-bit byte offsets, which run up to a block past the
    # last one, do not reach, so every m <= 32 takes the 64-bit staged path
    # (and the prefill GEMM addresses weights with 64-bit pointers).  Packed
    # tensors are drawn directly (random nibbles, steps and zeros); outputs are
    # checked on sampled columns, the ragged end among them.
    n, k, g = (1 << 20) - 5, 8192, 128
    gen = torch.Generator(device=DEV).manual_seed(620)
    qw = torch.randint(-2**31, 2**31 - 1, (n, k // 8), dtype=torch.int32, device=DEV, generator=gen)
    sc = (torch.rand((n, k // g), device=DEV, generator=gen) * 0.01 + 0.001).half()
    qz = torch.randint(-2**31, 2**31 - 1, (n, k // (8 * g)), dtype=torch.int32, device=DEV, generator=gen)
    xc = S.activations(64, k, 621, S.outlier_channels(k, 0.01, 622), 20.0)
    inv = O.fp16_rn(1.0 / O.scale_candidate(O.calib_stats(xc), 0.4).astype(np.float64))
    rng = np.random.Generator(np.random.PCG64(623))
    cols = np.unique(np.concatenate([rng.choice(n, 96, replace=False), np.arange(n - 21, n),
                                     np.arange((1 << 20) - 40, (1 << 20) - 30)]))
    ci = torch.from_numpy(cols).to(DEV)
    hq, hs, hz = host_u32(qw[ci]), sc[ci].cpu().numpy(), host_u32(qz[ci])
    for m in (1, 8, 24, 40):
        x = S.activations(m, k, 624 + m, S.outlier_channels(k, 0.01, 622), 20.0)
        y = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=g)
        torch.cuda.synchronize()
        yr = O.linear_ref(x, hq, hs, hz, inv, k, g)
        ok, worst, raw = O.check_linear(host16(y[:, ci]), yr)
        assert ok, (m, worst, raw)
        del y


@pytest.mark.parametrize("m", [33, 64, 256, 300])
def test_linear_split_k_full_size_sampled(P, m):
    # between the skinny kernels and a full prefill the GEMM's tiles alone
    # leave CUs idle: 64-row tiles up to 64 tokens, and each tile's K-steps
    # split over several work-groups (fp32 partial tiles in the workspace, summed in
    # slice order by a second launch).  Full Llama-3-8B shapes, sampled
    # columns against the oracle, and a second call bit for bit equal.
    rng = np.random.Generator(np.random.PCG64(700 + m))
    for n, k, alpha in ((4096, 4096, 0.5), (1024, 4096, 0.3), (4096, 14336, 0.45)):
        w = S.weights(n, k, 0.02, 701 + n + k)
        xc = S.activations(64, k, 702 + k, S.outlier_channels(k, 0.01, 703), 20.0)
        s16 = O.scale_candidate(O.calib_stats(xc), alpha)
        inv = O.fp16_rn(1.0 / s16.astype(np.float64))
        (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, s16, 128)
        del w
        x = S.activations(m, k, 704 + m + k, S.outlier_channels(k, 0.01, 703), 20.0)
        y = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=128)
        y2 = P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=128)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        cols = np.unique(np.concatenate([rng.choice(n, 96, replace=False), np.arange(n - 8, n)]))
        yr = O.linear_ref_rows(x, hq, hs, hz, inv, k, 128, cols)
        ok, worst, raw = O.check_linear(host16(y)[:, cols], yr)
        assert ok, (m, n, k, worst, raw)


@pytest.mark.parametrize("m,k,g", [(40, 14336, 32), (300, 14336, 32), (2048, 28672, 32), (64, 28672, 64)])
def test_linear_gemm_long_k_small_groups(P, m, k, g):
    # the scales and zero words of a tile's whole K range exceed LDS (K / g up
    # to 896 groups): the GEMM splits K until one slice's groups fit, at any m
    n = 264
    w = S.weights(n, k, 0.02, 720 + k // g)
    xc = S.activations(64, k, 721, S.outlier_channels(k, 0.01, 722), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.35)
    x = S.activations(m, k, 723 + m, S.outlier_channels(k, 0.01, 722), 20.0)
    cols = np.unique(np.concatenate([np.arange(0, 8), np.arange(128, 136), np.arange(n - 8, n)]))
    _check_linear(P, w, x, s16, g, cols=None if m <= 300 else cols)


def test_linear_split_k_graph_replays(P):
    # a captured split-K call (GEMM launch + slice-sum launch over workspace
    # partials) replayed several times, with eager calls of other sizes in
    # between that reuse the same workspace: every replay matches the eager result
    k, n, m = 4096, 1024, 64
    w = S.weights(n, k, 0.02, 710)
    qw, sc, qz, _ = P.awq_pack_int4(dev(w), None, g=128)
    x = dev(S.activations(m, k, 711, S.outlier_channels(k, 0.01, 712), 20.0))
    x_other = dev(S.activations(40, k, 713, S.outlier_channels(k, 0.01, 712), 20.0))
    need = max(P.awq_linear_workspace_size(m, n, k, 128), P.awq_linear_workspace_size(40, n, k, 128))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y_eager = P.awq_linear_w4a16(x, qw, sc, qz, None, g=128, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gr, stream=stream):
            P.awq_linear_w4a16(x, qw, sc, qz, None, g=128, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), i
        y_mid = P.awq_linear_w4a16(x_other, qw, sc, qz, None, g=128, workspace=ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(y_mid).all())


# ----------------------------------------------------------------- linear groups


def _group_case(P, m, k, g, specs, seed):
    """Linears (n, alpha or None, seed) reading two inputs; returns the group
    items and, per linear, its host packed tensors, inv_s16 and input."""
    xa = S.activations(m, k, seed, S.outlier_channels(k, 0.01, seed + 1), 20.0)
    xb = S.activations(m, k, seed + 2, S.outlier_channels(k, 0.01, seed + 1), 20.0)
    xs = [(dev(xa), xa), (dev(xb), xb)]
    items, meta = [], []
    for i, (n, alpha, sd) in enumerate(specs):
        w = S.weights(n, k, 0.02, sd)
        if alpha is None:
            s16 = inv = None
        else:
            xc = S.activations(64, k, sd + 1, S.outlier_channels(k, 0.01, sd + 2), 20.0)
            s16 = O.scale_candidate(O.calib_stats(xc), alpha)
            inv = O.fp16_rn(1.0 / s16.astype(np.float64))
        (qw, sc, qz), host = oracle_pack(w, s16, g)
        del w
        x_d, x_h = xs[i % 2]
        inv_d = None if inv is None else dev(inv)
        items.append((x_d, qw, sc, qz, inv_d, None))
        meta.append((x_d, x_h, qw, sc, qz, inv, inv_d, host))
    return items, meta


def _check_group(P, items, meta, k, g, cols_per=None):
    ys = P.awq_linear_w4a16_group(items, g=g)
    for y, (x_d, x_h, qw, sc, qz, inv, inv_d, host) in zip(ys, meta):
        y1 = P.awq_linear_w4a16(x_d, qw, sc, qz, inv_d, g=g)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
        n = qw.shape[0]
        hq, hs, hz = host
        if cols_per is None or n <= cols_per:
            yr = O.linear_ref(x_h, hq, hs, hz, inv, k, g)
            ok, worst, raw = O.check_linear(host16(y), yr)
        else:
            cols = np.sort(np.random.Generator(np.random.PCG64(n + 5)).choice(n, cols_per, replace=False))
            yr = O.linear_ref_rows(x_h, hq, hs, hz, inv, k, g, cols)
            ok, worst, raw = O.check_linear(host16(y)[:, cols], yr)
        assert ok, (n, worst, raw)


@pytest.mark.parametrize("m", [1, 8, 24, 40, 300])
@pytest.mark.parametrize("g", [128, 64])
def test_linear_group_matches_single_and_oracle(P, m, g):
    # m = 1, 8 and 24: one grouped decode launch (at 24 the group-major kernel
    # with two token chunks);
    # m = 40 and 300 (two row tiles, the second ragged): one activation-prep
    # launch and one GEMM launch over the tiles of every linear
    specs = [(1000, 0.5, 460), (256, 0.3, 470), (264, None, 480), (16, 0.4, 490)]
    items, meta = _group_case(P, m, 2048, g, specs, 461 + m)
    _check_group(P, items, meta, 2048, g)
    _check_group(P, items[1:3], meta[1:3], 2048, g)


@pytest.mark.parametrize("m", [1, 8, 24, 2048])
def test_linear_group_llama3_8b_full_size_sampled(P, m):
    qkv = [(4096, 0.5, 500), (1024, 0.4, 510), (1024, 0.45, 520)]
    items, meta = _group_case(P, m, 4096, 128, qkv, 530 + m)
    _check_group(P, items, meta, 4096, 128, cols_per=128)
    gate_up = [(14336, 0.5, 540), (14336, 0.35, 550)]
    items, meta = _group_case(P, m, 4096, 128, gate_up, 560 + m)
    _check_group(P, items, meta, 4096, 128, cols_per=128)


@pytest.mark.parametrize("m", [8, 20, 32])
def test_linear_group_mixed_plan(P, m):
    # m = 8: the group takes two column blocks per work-group (group-major
    # kernel), the small linears alone take one (block-major kernel); above 16
    # tokens the linear of more than 16 MiB of packed weights in 896 column
    # blocks runs the grouped GEMM and the small linears share one launch of
    # the two-chunk group-major kernel
    specs = [(14336, 0.5, 570), (1024, 0.4, 580), (264, None, 590)]
    items, meta = _group_case(P, m, 4096, 128, specs, 600 + m)
    _check_group(P, items, meta, 4096, 128, cols_per=128)


# ----------------------------------------------------------------- shared scale, folded 1/s


def test_fold_inv_scale_bit_exact(P):
    r = np.random.Generator(np.random.PCG64(800))
    k = 4099
    v = (r.standard_normal(k) * 10.0 ** r.integers(-5, 4, k)).astype(np.float16)
    v[:5] = np.array([0.0, -0.0, 65504.0, 6e-8, -3e-5], np.float16)
    s16 = O.scale_candidate(np.abs(r.standard_normal(k)) * 10.0 ** r.integers(-4, 4, k), 0.8)
    s16[:3] = np.array([2.0 ** -14, 1.0, 300.0], np.float16)
    want = O.fold_inv_scale(v, s16)
    vd, sd = dev(v), dev(s16)
    got = P.awq_fold_inv_scale(vd, sd)
    P.awq_fold_inv_scale(vd, sd, out=vd)          # in place
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert np.array_equal(vd.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_shared_scale_stacked_qkv_full_size(P):
    # q, k and v of one Llama-3-8B-shaped layer read one input and share one s:
    # awq_search_scale on their weights stacked along N (6144 x 4096, 128
    # calibration tokens).  On the GPU its losses are the sums of the three
    # per-linear searches' losses; on sampled rows of each part the search
    # matches the oracle bit for bit; the stacked linear, run with inv_s16 absent
    # on activations produced with the folded weight fp16_rn(gamma / s), matches
    # the oracle on sampled columns.
    parts = [S.config_layer(2, nm, n, k, 128, 8, 0.02, 0.01, 20.0) for nm, n, k in S.LLAMA3_8B_LINEARS[:3]]
    x_cal, x_run = parts[0][1], parts[0][2]
    for p_ in parts[1:]:
        assert np.array_equal(p_[1], x_cal)        # one shared input
    wst = np.concatenate([p_[0] for p_ in parts])
    wd, xd = dev(wst), dev(x_cal)
    a = P.awq_calib_stats(xd)
    best, s16, inv, losses = P.awq_search_scale(wd, xd, a)
    sums = [P.awq_search_scale(dev(p_[0]), xd, a)[3] for p_ in parts]
    torch.cuda.synchronize()
    tot = sum(v.cpu().numpy() for v in sums)
    assert np.max(np.abs(tot - losses.cpu().numpy()) / tot) < 1e-12
    rows = np.concatenate([np.arange(0, 4096, 64), 4096 + np.arange(0, 1024, 32), 5120 + np.arange(0, 1024, 32)])
    _check_search(P, np.ascontiguousarray(wst[rows]), x_cal, 128, 20)
    # the full stack's choice: the first minimum of its losses, and its s16 the
    # oracle's candidate at that alpha
    gl = losses.cpu().numpy()
    assert int(best.item()) == O.select_best(gl)
    s16_want = O.scale_candidate(O.calib_stats(x_cal), O.alpha_grid(20)[int(best.item())])
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), s16_want.view(np.uint16))
    # the operation producing the input (weight gamma) absorbs 1/s
    r = np.random.Generator(np.random.PCG64(801))
    gamma = (1.0 + 0.1 * r.standard_normal(4096)).astype(np.float16)
    s16h = s16.cpu().numpy()
    gfold = P.awq_fold_inv_scale(dev(gamma), s16)
    torch.cuda.synchronize()
    assert np.array_equal(gfold.cpu().numpy().view(np.uint16), O.fold_inv_scale(gamma, s16h).view(np.uint16))
    # the linear runs on the oracle's fold and the oracle's pack of the stack
    x_tilde = O.fp16_rn(x_run.astype(np.float64) *
                        O.fold_inv_scale(gamma, s16_want).astype(np.float64)[None, :])
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(wst, s16_want, 128)
    y = P.awq_linear_w4a16(dev(x_tilde), qw, sc, qz, None, g=128)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([r.choice(6144, 192, replace=False), np.arange(4090, 4100), np.arange(6136, 6144)]))
    yr = O.linear_ref(x_tilde, hq[cols], hs[cols], hz[cols], None, 4096, 128)
    ok, worst, raw = O.check_linear(host16(y)[:, cols], yr)
    assert ok, (worst, raw)
    # the GPU pack of the stack at the shared s is the oracle's pack
    gq, gs, gz, _ = P.awq_pack_int4(wd, s16, g=128)
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(gq), hq)
    assert np.array_equal(gs.cpu().numpy().view(np.uint16), hs.view(np.uint16))
    assert np.array_equal(host_u32(gz), hz)


def test_fold_inv_scale_rows_bit_exact(P):
    r = np.random.Generator(np.random.PCG64(810))
    n, k = 37, 1031
    w = (r.standard_normal((n, k)) * 10.0 ** r.integers(-5, 4, (n, k))).astype(np.float16)
    w[0, :5] = np.array([0.0, -0.0, 65504.0, 6e-8, -3e-5], np.float16)
    s16 = O.scale_candidate(np.abs(r.standard_normal(n)) * 10.0 ** r.integers(-4, 4, n), 0.8)
    s16[:3] = np.array([2.0 ** -14, 1.0, 300.0], np.float16)
    want = O.fold_inv_scale_rows(w, s16)
    wd, sd = dev(w), dev(s16)
    got = P.awq_fold_inv_scale_rows(wd, sd)
    P.awq_fold_inv_scale_rows(wd, sd, out=wd)          # in place
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert np.array_equal(wd.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_fold_rows_up_for_down_full_size(P):
    # the down projection's s (its input has 14336 channels) folded into the
    # rows of the Llama-3-8B up projection (14336 x 4096): bit-exact on every
    # element, and the folded up projection's pack is the oracle's pack of the
    # folded weight on sampled rows
    _, x_cal, _, _ = S.config_layer(2, "down", 4096, 14336, 128, 0, 0.02, 0.01, 20.0)
    w_up = S.config_layer(2, "up", 14336, 4096, 8, 0, 0.02, 0.01, 20.0)[0]
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.45)
    got = P.awq_fold_inv_scale_rows(dev(w_up), dev(s16))
    torch.cuda.synchronize()
    want = O.fold_inv_scale_rows(w_up, s16)
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16))
    qw, sc, qz, _ = P.awq_pack_int4(got, None, g=128)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(811)).choice(14336, 64, replace=False))
    ri = torch.from_numpy(rows).to(DEV)
    oq, osc, oz = O.pack_int4(want[rows], None, 128)[:3]
    assert np.array_equal(host_u32(qw[ri]), oq)
    assert np.array_equal(sc[ri].cpu().numpy().view(np.uint16), osc.view(np.uint16))
    assert np.array_equal(host_u32(qz[ri]), oz)
