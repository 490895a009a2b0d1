"""GPU parity for the mixed-precision baseline (protected channels kept in
fp16, the rest RTN) against the CPU oracle: the protected channel indices, the
keep mask and the gathered columns bit-exact; the mixed loss within the search
loss's accumulation bound; the mixed linear within the floored relative
tolerance 5e-3 against float64."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O

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


# ----------------------------------------------------------------- selection


@pytest.mark.parametrize("k,count", [(1, 0), (1, 1), (7, 3), (1000, 10), (4096, 41), (14336, 143),
                                     (28672, 287), (3000, 1024), (1030, 1024)])
def test_salient_channels_bit_exact(P, k, count):
    r = np.random.Generator(np.random.PCG64(2600 + k + count))
    a = r.random(k) * 3.0
    a[r.choice(k, min(k, 40), replace=False)] = 1.5          # ties, some at the boundary
    if k > 10:
        a[r.choice(k, 3, replace=False)] = np.nan
        a[int(r.integers(0, k))] = np.inf
        a[int(r.integers(0, k))] = 0.0
        a[int(r.integers(0, k))] = -0.0
    got = P.awq_salient_channels(dev(a), count)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.salient_channels(a, count))


def test_salient_channels_all_equal(P):
    # every value equal: the lowest indices win
    a = np.full(5000, 0.25)
    got = P.awq_salient_channels(dev(a), 50)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), np.arange(50, dtype=np.int32))


def test_salient_channels_of_calibration(P):
    # the calibration statistic of the Llama-3-8B down projection's input
    k = 14336
    _, x_cal, _, ch = S.config_layer(3, "down", 4096, k, 512, 0, 0.02, 0.01, 20.0)
    a = P.awq_calib_stats(dev(x_cal))
    cnt = O.salient_count(k, 0.01)
    got = P.awq_salient_channels(a, cnt)
    torch.cuda.synchronize()
    want = O.salient_channels(O.calib_stats(x_cal), cnt)
    assert np.array_equal(got.cpu().numpy(), want)
    assert set(want.tolist()) <= set(ch.tolist())


def test_mask_and_gather_bit_exact(P):
    n, k = 37, 1000
    w = S.weights(n, k, 0.02, 2610)
    idx = np.sort(np.random.Generator(np.random.PCG64(2611)).choice(k, 13, replace=False)).astype(np.int32)
    keep = P.awq_channel_mask(dev(idx), k)
    ws = P.awq_gather_channels(dev(w), dev(idx))
    torch.cuda.synchronize()
    want = np.ones(k, np.float16)
    want[idx] = 0
    assert np.array_equal(keep.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert np.array_equal(ws.cpu().numpy().view(np.uint16), np.ascontiguousarray(w[:, idx].T).view(np.uint16))


# ----------------------------------------------------------------- loss


def _check_mixed_loss(P, w, x, idx, g):
    keep = P.awq_channel_mask(dev(idx), w.shape[1])
    got = float(P.awq_mixed_loss(dev(w), dev(x), keep, g=g).item())
    want = O.mixed_loss(w, x, idx, g)
    # the search kernel's accumulation bound on the masked activations
    gamma = 1e-5
    xm = x.astype(np.float64)
    xm[:, idx] = 0
    dw = O.mixed_weight(w, idx, g) - w.astype(np.float64)
    sabs = float(np.sum((np.abs(dw) @ np.abs(xm).T) ** 2))
    bound = 2 * gamma * np.sqrt(want * sabs) + gamma * gamma * sabs
    assert abs(got - want) <= bound, (got, want, bound)
    return got, want


@pytest.mark.parametrize("n,k,m,g", [(40, 256, 20, 64), (70, 384, 130, 128), (33, 96, 5, 32)])
def test_mixed_loss_small(P, n, k, m, g):
    ch = S.outlier_channels(k, 0.02, 2621)
    w = S.weights(n, k, 0.02, 2620 + n)
    x = S.activations(m, k, 2622 + m, ch, 20.0)
    idx = O.salient_channels(O.calib_stats(x), O.salient_count(k, 0.02))
    _check_mixed_loss(P, w, x, idx, g)
    _check_mixed_loss(P, w, x, np.zeros(0, np.int32), g)


def test_mixed_loss_full_k_sampled_rows(P):
    # the Llama-3-8B q projection with 512 calibration tokens on 64 rows, 1 % protected
    n, k = 4096, 4096
    w, x_cal, _, _ = S.config_layer(3, "q", n, k, 512, 0, 0.02, 0.01, 20.0)
    rows = np.sort(np.random.Generator(np.random.PCG64(2630)).choice(n, 64, replace=False))
    idx = O.salient_channels(O.calib_stats(x_cal), O.salient_count(k, 0.01))
    got, want = _check_mixed_loss(P, np.ascontiguousarray(w[rows]), x_cal, idx, 128)
    # protecting the outlier channels cuts the plain RTN loss
    rtn = O.search_loss(w[rows], x_cal, np.ones(k, np.float16), 128)
    assert want < rtn


# ----------------------------------------------------------------- linear


def _check_mixed_linear(P, w, x, idx, g, cols=None):
    k = w.shape[1]
    hq, hs, hz, _ = O.pack_int4(w, None, g)          # the oracle's RTN pack, uploaded
    qw, sc, qz = dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32))
    di = dev(idx)
    keep = P.awq_channel_mask(di, k)
    ws = P.awq_gather_channels(dev(w), di)
    y = P.awq_linear_mixed(dev(x), qw, sc, qz, keep, ws, di, g=g)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    if cols is None:
        yr = O.linear_mixed_ref(x, hq, hs, hz, w, idx, k, g)
        ok, worst, raw = O.check_linear(yh, yr)
    else:
        yr = O.linear_mixed_ref(x, hq[cols], hs[cols], hz[cols], w[cols], idx, k, g)
        ok, worst, raw = O.check_linear(yh[:, cols], yr)
    assert ok, (worst, raw)


@pytest.mark.parametrize("m", [1, 5, 16, 17, 33, 300])
@pytest.mark.parametrize("g", [32, 128])
def test_linear_mixed_small(P, m, g):
    n, k = 300, 640
    ch = S.outlier_channels(k, 0.02, 2641)
    w = S.weights(n, k, 0.02, 2640 + m)
    x = S.activations(m, k, 2642 + m, ch, 30.0)
    idx = O.salient_channels(O.calib_stats(S.activations(64, k, 2643, ch, 30.0)), O.salient_count(k, 0.02))
    _check_mixed_linear(P, w, x, idx, g)
    _check_mixed_linear(P, w, x, np.zeros(0, np.int32), g)


def test_linear_mixed_many_protected(P):
    # 1024 protected channels (the limit): the add pass's LDS takes 92 KiB
    n, k, g = 130, 4096, 128
    w = S.weights(n, k, 0.02, 2660)
    idx = np.sort(np.random.Generator(np.random.PCG64(2661)).choice(k, 1024, replace=False)).astype(np.int32)
    for m in (1, 20):
        x = S.activations(m, k, 2662 + m)
        _check_mixed_linear(P, w, x, idx, g)


@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
def test_linear_mixed_decode_full_size(P, name, n, k):
    w, x_cal, x_run, _ = S.config_layer(2, name, n, k, 128, 1, 0.02, 0.01, 20.0)
    idx = O.salient_channels(O.calib_stats(x_cal), O.salient_count(k, 0.01))
    _check_mixed_linear(P, w, x_run, idx, 128)


def test_linear_mixed_prefill_sampled(P):
    n, k = 4096, 14336
    w, x_cal, x_run, _ = S.config_layer(3, "down", n, k, 512, 2048, 0.02, 0.01, 20.0)
    idx = O.salient_channels(O.calib_stats(x_cal), O.salient_count(k, 0.01))
    cols = np.sort(np.random.Generator(np.random.PCG64(2650)).choice(n, 48, replace=False))
    _check_mixed_linear(P, w, x_run, idx, 128, cols=cols)
