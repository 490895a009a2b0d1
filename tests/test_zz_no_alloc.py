"""awq_linear_w4a16_group_noalloc (no workspace, nothing allocated: the scratch
is a static device array of the library) through the C ABI, against
awq_linear_w4a16_group with a caller workspace: bit-identical outputs on two
calls in a row, the second with fewer tokens (the array keeps the first
call's contents), and both within the oracle's tolerance.  A call whose plan
needs more than the static array is refused before any launch."""
from __future__ import annotations

import ctypes as C

import numpy as np
import pytest

import synthetic as S
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import weight_only_int4_awq_amd as P
    lib = P.load()
    assert torch.cuda.is_available()
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _items(linears, x, m):
    from weight_only_int4_awq_amd import _lib
    arr = (_lib.LinearItem * len(linears))()
    outs = []
    for i, (qw, sc, qz, inv, n) in enumerate(linears):
        y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
        a = arr[i]
        a.x, a.inv_s16, a.qweight, a.scales, a.qzeros, a.y, a.n = (
            x.data_ptr(), inv.data_ptr(), qw.data_ptr(), sc.data_ptr(), qz.data_ptr(), y.data_ptr(), n)
        outs.append(y)
    return arr, outs


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_noalloc_group_matches_workspace_call(lib):
    k, g = 2048, 128
    ch = S.outlier_channels(k, 0.01, 1901)
    linears, hosts = [], []
    for i, n in enumerate((1000, 264, 520)):
        w = S.weights(n, k, 0.02, 1902 + i)
        s16 = O.scale_candidate(O.calib_stats(S.activations(64, k, 1905 + i, ch, 20.0)), 0.35 + 0.05 * i)
        inv = O.fp16_rn(1.0 / s16.astype(np.float64))
        hq, hs, hz, _ = O.pack_int4(w, s16, g)
        linears.append((dev(hq.view(np.int32)), dev(hs), dev(hz.view(np.int32)), dev(inv), n))
        hosts.append(((hq, hs, hz), inv))
    ns = (C.c_int64 * 3)(*[lin[4] for lin in linears])
    assert lib.awq_linear_noalloc_scratch_bytes() == 64 << 20
    # 600 tokens (GEMM: x_tilde slots, three row tiles), then 256 (split-K
    # GEMM: slots and partial tiles), 40 (64-row split-K tiles), 24 (two-chunk
    # group-major kernel, no scratch), 8 (token-row decode GEMV, no scratch)
    # and 1; every plan fits the static scratch
    for m in (600, 256, 40, 24, 8, 1):
        x_h = S.activations(m, k, 1910 + m, ch, 20.0)
        x = dev(x_h)
        need = lib.awq_linear_group_workspace_size(ns, 3, m, k, g)
        assert need <= lib.awq_linear_noalloc_scratch_bytes(), (m, need)
        arr_a, out_a = _items(linears, x, m)
        st = lib.awq_linear_w4a16_group_noalloc(arr_a, 3, m, k, g, _stream())
        assert st == 0, lib.awq_last_error().decode()
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        arr_b, out_b = _items(linears, x, m)
        st = lib.awq_linear_w4a16_group(arr_b, 3, m, k, g, C.c_void_p(ws.data_ptr() if need else None),
                                        need, _stream())
        assert st == 0, lib.awq_last_error().decode()
        torch.cuda.synchronize()
        for ya, yb, (host, inv) in zip(out_a, out_b, hosts):
            assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), m
            ok, worst, raw = O.check_linear(ya.cpu().numpy(), O.linear_ref(x_h, *host, inv, k, g))
            assert ok, (m, worst, raw)


def test_noalloc_refuses_plans_beyond_the_static_scratch(lib):
    # the 70B-shaped down projection at 2048 tokens stages 112 MiB of x_tilde:
    # refused on the host, nothing launched (the pointers are never read)
    from weight_only_int4_awq_amd import _lib
    n, k, m = 8192, 28672, 2048
    ns = (C.c_int64 * 1)(n)
    assert lib.awq_linear_group_workspace_size(ns, 1, m, k, 128) > lib.awq_linear_noalloc_scratch_bytes()
    arr = (_lib.LinearItem * 1)()
    a = arr[0]
    a.x = a.qweight = a.scales = a.qzeros = a.y = 0x10000
    a.inv_s16 = None
    a.n = n
    st = lib.awq_linear_w4a16_group_noalloc(arr, 1, m, k, 128, None)
    assert st == 4
    assert "static scratch" in lib.awq_last_error().decode()
