"""GPU parity for bf16 activations (awq_linear_w4a16_bf16 and its group call)
against the CPU oracle: outputs within the floored relative tolerance 5e-3
against float64 on every decode plan (GEMV, fused and group-major skinny,
prep16 + skinny16, staged pair) and the GEMM (with and without split-K).
Structural checks: the group call writes the single calls' bits, and the bf16
result and the fp16 result of the same (fp16-exact) activations are two
roundings of one fp32 value."""
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


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bf16(t):
    return O.bf16_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def _pack(P, w, s16, g):
    """The oracle's pack of w at s16, uploaded (linear tests never feed the
    oracle a GPU result)."""
    hq, hs, hz, _ = O.pack_int4(w, s16, g)
    return dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32)), (hq, hs, hz)


def _check(P, w, xb, s16, g, cols=None):
    """bf16 linear against the oracle; returns (y bf16 as float64, packed tensors, inv)."""
    inv = None if s16 is None else O.fp16_rn(1.0 / s16.astype(np.float64))
    qw, sc, qz, (hq, hs, hz) = _pack(P, w, s16, g)
    y = P.awq_linear_w4a16_bf16(dev_bf16(xb), qw, sc, qz, None if inv is None else dev(inv), g=g)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    k = w.shape[1]
    x = O.bf16_to_f64(xb)
    yh = host_bf16(y)
    if cols is None:
        yr = O.linear_ref(x, hq, hs, hz, inv, k, g)
        ok, worst, raw = O.check_linear(yh, yr)
    else:
        yr = O.linear_ref_rows(x, hq, hs, hz, inv, k, g, cols)
        ok, worst, raw = O.check_linear(yh[:, cols], yr)
    assert ok, (worst, raw)
    return yh, (qw, sc, qz), inv


@pytest.mark.parametrize("m", [1, 2, 8, 16, 17, 31, 32, 33, 100, 257])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_linear_bf16_small(P, m, g):
    n, k = 50, 640
    w = S.weights(n, k, 0.02, 2400 + m)
    xb = S.activations_bf16(m, k, 2401 + m, S.outlier_channels(k, 0.01, 2402), 20.0)
    xc = S.activations(64, k, 2403, S.outlier_channels(k, 0.01, 2402), 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), 0.4)
    _check(P, w, xb, s16, g)
    _check(P, w, xb, None, g)


@pytest.mark.parametrize("m", [1, 8, 20, 40])
def test_linear_bf16_matches_fp16_rounding(P, m):
    # bf16 activations are exact in fp16 here, so both calls accumulate the
    # same fp32 value: the bf16 and fp16 outputs are its two roundings
    n, k, g = 257, 1152, 128
    w = S.weights(n, k, 0.02, 2410)
    xb = S.activations_bf16(m, k, 2411 + m, S.outlier_channels(k, 0.01, 2412), 20.0)
    xb[np.abs(O.bf16_to_f64(xb)) < 2.0 ** -14] = 0          # below the fp16 normal range
    x = O.bf16_to_f64(xb)
    xh = x.astype(np.float16)
    assert np.array_equal(xh.astype(np.float64), x)
    yb, (qw, sc, qz), _ = _check(P, w, xb, None, g)
    yh = P.awq_linear_w4a16(dev(xh), qw, sc, qz, None, g=g).cpu().numpy().astype(np.float64)
    fin = np.isfinite(yh) & np.isfinite(yb)
    assert fin.all()
    # |y_bf16 - y_fp16| <= half an ulp of each format at that magnitude
    mag = np.maximum(np.abs(yb), np.abs(yh))
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -126)))
    bound = 2.0 ** (e - 8) + 2.0 ** (np.maximum(e, -14) - 11)
    assert np.all(np.abs(yb - yh) <= bound * 1.0000001)


@pytest.mark.parametrize("name,n,k", S.LLAMA3_8B_LINEARS)
@pytest.mark.parametrize("m", [1, 8])
def test_linear_bf16_decode_full_size(P, name, n, k, m):
    w, x_cal, _, ch = S.config_layer(2, name, n, k, 128, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    xb = S.activations_bf16(m, k, 2420 + m + n, ch, 20.0)
    _check(P, w, xb, s16, 128)


@pytest.mark.parametrize("m", [20, 32, 2048])
def test_linear_bf16_gate_up_full_size(P, m):
    # m = 20 and 32: the wide-linear GEMM of the decode plan; 2048: prefill
    n, k = 14336, 4096
    w, x_cal, _, ch = S.config_layer(3, "gate", n, k, 512, 0, 0.02, 0.01, 20.0)
    s16 = O.scale_candidate(O.calib_stats(x_cal), 0.4)
    xb = S.activations_bf16(m, k, 2430 + m, ch, 20.0)
    cols = np.sort(np.random.Generator(np.random.PCG64(2431 + m)).choice(n, 64, replace=False))
    _check(P, w, xb, s16, 128, cols=cols)


@pytest.mark.parametrize("m", [1, 8, 24])
def test_linear_bf16_staged_wide_k(P, m):
    # k = 65536: the GEMV, fused and prep16 plans do not fit LDS, the staged
    # two-kernel path runs at every m
    n, k, g = 16, 65536, 128
    w = S.weights(n, k, 0.015, 2440)
    xb = S.activations_bf16(m, k, 2441 + m, S.outlier_channels(k, 0.005, 2442), 30.0)
    _check(P, w, xb, None, g)


def test_linear_bf16_decode_multiblock(P):
    # several column blocks per work-group of the GEMV and of the group-major
    # skinny kernel (m = 1 and 4)
    n, k, g = 12345, 2048, 32
    w = S.weights(n, k, 0.02, 2445)
    for m in (1, 4):
        xb = S.activations_bf16(m, k, 2446 + m, S.outlier_channels(k, 0.01, 2447), 20.0)
        _check(P, w, xb, None, g)


@pytest.mark.parametrize("m", [1, 4, 24, 300])
def test_linear_bf16_group_matches_single(P, m):
    k, g = 4096, 128
    ns = (1024, 512, 512)
    xb = dev_bf16(S.activations_bf16(m, k, 2450 + m, S.outlier_channels(k, 0.01, 2451), 20.0))
    inv = dev(O.fp16_rn(1.0 / O.scale_candidate(
        O.calib_stats(S.activations(64, k, 2452, S.outlier_channels(k, 0.01, 2451), 20.0)), 0.3)
        .astype(np.float64)))
    packs = [_pack(P, S.weights(n, k, 0.02, 2453 + i), None, g)[:3] for i, n in enumerate(ns)]
    singles = [P.awq_linear_w4a16_bf16(xb, qw, sc, qz, inv, g=g) for qw, sc, qz in packs]
    outs = P.awq_linear_w4a16_group_bf16([(xb, qw, sc, qz, inv, None) for qw, sc, qz in packs], g=g)
    torch.cuda.synchronize()
    for a, b in zip(singles, outs):
        assert b.dtype == torch.bfloat16
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_linear_bf16_deterministic(P):
    w = S.weights(512, 2048, 0.02, 2461)
    qw, sc, qz, _ = _pack(P, w, None, 128)
    for m in (1, 8, 32, 300):
        xb = dev_bf16(S.activations_bf16(m, 2048, 2462 + m))
        a = P.awq_linear_w4a16_bf16(xb, qw, sc, qz, None, g=128)
        b = P.awq_linear_w4a16_bf16(xb, qw, sc, qz, None, g=128)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
