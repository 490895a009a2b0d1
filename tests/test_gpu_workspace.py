"""GPU checks of the linear calls' memory contract: every output and every
caller workspace sits inside a sentinel-filled guard band, and after the call
the bands are unchanged (no write past an output's end, a ragged last block,
a split-K partial tile or the workspace size the query returned); calls on two
streams with workspaces of their own give the bits of one stream; a first
call can be captured in a graph (the library allocates nothing).  Outputs are
checked against the oracle (packed weights from the oracle's pack)."""
from __future__ import annotations

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
GUARD = 4096            # bytes of sentinel before and after each region
SENT = 0x5A


@pytest.fixture(scope="module")
def P():
    import weight_only_int4_awq_amd as P
    P.load()
    assert torch.cuda.is_available()
    return P


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def oracle_pack(w, s16, g, w_bit=4):
    hq, hs, hz, _ = O.pack_weights(w, s16, g, w_bit)
    return (dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32))), (hq, hs, hz)


class Guarded:
    """A region of `nbytes` inside a sentinel-filled buffer (256-byte aligned)."""

    def __init__(self, nbytes):
        self.nbytes = nbytes
        self.buf = torch.full((GUARD + max(nbytes, 1) + GUARD,), SENT, dtype=torch.uint8, device=DEV)
        self.region = self.buf[GUARD:GUARD + nbytes]

    def view(self, dtype, shape):
        return self.region.view(dtype).view(shape)

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool((b[:GUARD] == SENT).all() and (b[GUARD + self.nbytes:] == SENT).all())


def _case(n, k, m, seed, alpha=0.4):
    w = S.weights(n, k, 0.02, seed)
    ch = S.outlier_channels(k, 0.01, seed + 1)
    xc = S.activations(64, k, seed + 2, ch, 20.0)
    s16 = O.scale_candidate(O.calib_stats(xc), alpha)
    inv = O.fp16_rn(1.0 / s16.astype(np.float64))
    x = S.activations(m, k, seed + 3, ch, 20.0)
    return w, s16, inv, x


def _check_rows(y_host, x, host, inv, k, g, w_bit=4):
    yr = O.linear_ref(x, *host, inv, k, g, w_bit)
    ok, worst, raw = O.check_linear(y_host, yr)
    assert ok, (worst, raw)


# (n, k, m, g): m = 1 decode GEMV with a ragged last block; 8 fused skinny;
# 24 two-chunk group-major kernel (also on 16.4 MiB of packed weights in 257
# blocks, the last ragged); 24 on a linear above 16 MiB in more than 512 blocks
# (grouped GEMM with 64-row tiles split along K); 33 and 64 split-K GEMM; 300
# GEMM with a ragged second row tile; k = 65536 the staged two-kernel decode path
CASES = [(1000, 2048, 1, 128), (1000, 2048, 8, 64), (257, 4096, 24, 128), (4100, 8192, 24, 128),
         (8200, 4096, 24, 128),
         (1000, 2048, 33, 128), (1000, 4096, 64, 32), (260, 2048, 300, 128), (40, 65536, 8, 128)]


@pytest.mark.parametrize("n,k,m,g", CASES)
def test_linear_guard_bands(P, n, k, m, g):
    w, s16, inv, x = _case(n, k, m, 900 + n + m)
    (qw, sc, qz), host = oracle_pack(w, s16, g)
    need = P.awq_linear_workspace_size(m, n, k, g)
    wsg = Guarded(need)
    yg = Guarded(m * n * 2)
    y = yg.view(torch.float16, (m, n))
    P.awq_linear_w4a16(dev(x), qw, sc, qz, dev(inv), g=g, out=y,
                       workspace=wsg.region if need else None)
    torch.cuda.synchronize()
    assert yg.intact(), "write outside y"
    assert wsg.intact(), "write outside the workspace"
    _check_rows(y.cpu().numpy(), x, host, inv, k, g)


@pytest.mark.parametrize("m", [1, 8, 24, 40])
def test_linear_group_guard_bands(P, m):
    k, g = 2048, 128
    specs = [(1000, 930), (264, 931), (8200 * 2, 932)]   # the last above 16 MiB at k = 2048
    ch = S.outlier_channels(k, 0.01, 933)
    x = S.activations(m, k, 934 + m, ch, 20.0)
    xd = dev(x)
    items, metas, guards = [], [], []
    for n, sd in specs:
        w = S.weights(n, k, 0.02, sd)
        s16 = O.scale_candidate(O.calib_stats(S.activations(64, k, sd + 1, ch, 20.0)), 0.35)
        inv = O.fp16_rn(1.0 / s16.astype(np.float64))
        (qw, sc, qz), host = oracle_pack(w, s16, g)
        yg = Guarded(m * n * 2)
        items.append((xd, qw, sc, qz, dev(inv), yg.view(torch.float16, (m, n))))
        metas.append((host, inv))
        guards.append(yg)
    need = P.awq_linear_group_workspace_size([n for n, _ in specs], m, k, g)
    wsg = Guarded(need)
    ys = P.awq_linear_w4a16_group(items, g=g, workspace=wsg.region if need else None)
    torch.cuda.synchronize()
    assert wsg.intact()
    for y, yg, (host, inv) in zip(ys, guards, metas):
        assert yg.intact()
        _check_rows(y.cpu().numpy(), x, host, inv, k, g)


@pytest.mark.parametrize("w_bit", [3, 8])
@pytest.mark.parametrize("m", [1, 16, 24, 64])
def test_linear_wbit_guard_bands(P, w_bit, m):
    n, k, g = 1000, 2048, 128
    w, s16, inv, x = _case(n, k, m, 940 + m + w_bit)
    (qw, sc, qz), host = oracle_pack(w, s16, g, w_bit)
    need = P.awq_linear_wbit_workspace_size(m, n, k, g, w_bit, True)
    wsg = Guarded(need)
    yg = Guarded(m * n * 2)
    y = yg.view(torch.float16, (m, n))
    P.awq_linear_wbit(dev(x), qw, sc, qz, dev(inv), g=g, w_bit=w_bit, out=y,
                      workspace=wsg.region if need else None)
    torch.cuda.synchronize()
    assert yg.intact() and wsg.intact()
    _check_rows(y.cpu().numpy(), x, host, inv, k, g, w_bit)


def test_linear_mixed_guard_bands(P):
    n, k, g, m = 1000, 2048, 128, 40
    w, _, _, x = _case(n, k, m, 950)
    a = O.calib_stats(S.activations(64, k, 951, S.outlier_channels(k, 0.01, 951), 20.0))
    idx = O.salient_channels(a, O.salient_count(k, 0.01))
    (qw, sc, qz), (hq, hs, hz) = oracle_pack(w, None, g)
    di = dev(idx.astype(np.int32))
    keep = P.awq_channel_mask(di, k)
    w_s = P.awq_gather_channels(dev(w), di)
    need = P.awq_linear_workspace_size(m, n, k, g)
    assert need > 0
    wsg = Guarded(need)
    yg = Guarded(m * n * 2)
    y = yg.view(torch.float16, (m, n))
    P.awq_linear_mixed(dev(x), qw, sc, qz, keep, w_s, di, g=g, out=y, workspace=wsg.region)
    torch.cuda.synchronize()
    assert yg.intact() and wsg.intact()
    yr = O.linear_mixed_ref(x, hq, hs, hz, w, idx, k, g)
    ok, worst, raw = O.check_linear(y.cpu().numpy(), yr)
    assert ok, (worst, raw)


@pytest.mark.parametrize("m", [8, 33, 64])
def test_linear_two_streams_own_workspaces(P, m):
    # the same call on two streams at once, each with a workspace of its own,
    # gives the bits of the call alone
    n, k, g = 4096, 4096, 128
    w, s16, inv, x = _case(n, k, m, 960 + m)
    (qw, sc, qz), host = oracle_pack(w, s16, g)
    xd, invd = dev(x), dev(inv)
    need = P.awq_linear_workspace_size(m, n, k, g)
    ref = P.awq_linear_w4a16(xd, qw, sc, qz, invd, g=g)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((m, n), dtype=torch.float16, device=DEV) for _ in range(2)]
    wss = [torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) for _ in range(2)]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for s, o, ws in zip(streams, outs, wss):
            with torch.cuda.stream(s):
                for _ in range(4):
                    P.awq_linear_w4a16(xd, qw, sc, qz, invd, g=g, out=o, workspace=ws if need else None)
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), rep
    _check_rows(ref.cpu().numpy(), x, host, inv, k, g)


@pytest.mark.parametrize("m", [1, 24, 64, 2048])
def test_linear_first_call_captured(P, m):
    # no eager call before the capture: nothing for the library to allocate
    n, k, g = 1024, 4096, 128
    w, s16, inv, x = _case(n, k, m, 970 + m)
    (qw, sc, qz), host = oracle_pack(w, s16, g)
    xd, invd = dev(x), dev(inv)
    need = P.awq_linear_workspace_size(m, n, k, g)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((m, n), dtype=torch.float16, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gr, stream=stream):
            P.awq_linear_w4a16(xd, qw, sc, qz, invd, g=g, out=out, workspace=ws if need else None)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    first = None
    for i in range(3):
        out.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        if first is None:
            first = out.clone()
            cols = np.unique(np.concatenate([np.arange(0, 64), np.arange(n - 64, n)]))
            yr = O.linear_ref_rows(x, *host, inv, k, g, cols)
            ok, worst, raw = O.check_linear(out.cpu().numpy()[:, cols], yr)
            assert ok, (worst, raw)
        else:
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), i
        # eager work of another size between the replays
        P.awq_linear_w4a16(dev(x[:1]), qw, sc, qz, invd, g=g)
        torch.cuda.synchronize()
