"""The C ABI library loads and exports every symbol the header declares, and its
host-side argument checks reject bad calls before any launch (CPU only: every
call here fails validation, so nothing reaches the GPU)."""
from __future__ import annotations

import ctypes as C
import pathlib
import re
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "awq_mi355x.h"


@pytest.fixture(scope="module")
def lib():
    from weight_only_int4_awq_amd import _lib
    if not _lib.LIB_PATH.exists():
        from weight_only_int4_awq_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = HEADER.read_text()
    body = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(awq_\w+)\s*\(", body, flags=re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for want in ("awq_calib_stats", "awq_search_scale", "awq_search_workspace_size",
                 "awq_pack_int4", "awq_linear_w4a16", "awq_linear_w4a16_group", "awq_fold_inv_scale",
                 "awq_search_scale_wbit", "awq_pack_wbit", "awq_linear_wbit",
                 "awq_linear_w4a16_bf16", "awq_linear_w4a16_group_bf16",
                 "awq_salient_channels", "awq_channel_mask", "awq_gather_channels",
                 "awq_mixed_loss_workspace_size", "awq_mixed_loss", "awq_linear_mixed",
                 "awq_fold_inv_scale_rows", "awq_last_error", "awq_abi_version",
                 "awq_linear_workspace_size", "awq_linear_group_workspace_size",
                 "awq_linear_wbit_workspace_size"):
        assert want in names, names


def test_library_exports_every_declared_symbol(lib):
    from weight_only_int4_awq_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
        assert name in _lib.SIGNATURES, name
    assert lib.awq_abi_version() == 2


FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = 0x10002


def _status(lib, fn, *args):
    st = getattr(lib, fn)(*args)
    msg = lib.awq_last_error().decode()
    return st, msg


def test_calib_stats_argument_errors(lib):
    assert _status(lib, "awq_calib_stats", None, 4, 64, FAKE, None)[0] == 1
    assert _status(lib, "awq_calib_stats", FAKE, 0, 64, FAKE, None)[0] == 2
    assert _status(lib, "awq_calib_stats", FAKE, 8193, 64, FAKE, None)[0] == 2
    assert _status(lib, "awq_calib_stats", FAKE, 4, 60, FAKE, None)[0] == 2
    st, msg = _status(lib, "awq_calib_stats", MISALIGNED, 4, 64, FAKE, None)
    assert st == 3 and "aligned" in msg


def test_search_argument_errors(lib):
    ws = lib.awq_search_workspace_size(64, 256, 16, 128, 20)
    assert ws > 0
    assert lib.awq_search_workspace_size(64, 256, 16, 96, 20) == 0
    assert lib.awq_search_workspace_size(64, 256, 16, 128, 65) == 0
    base = [FAKE, FAKE, FAKE, 64, 256, 16, 128, 20, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]

    def call(**kw):
        a = list(base)
        names = ["w", "x", "a", "n", "k", "m", "g", "ng", "best", "s", "inv", "loss", "ws", "wsb", "st"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_search_scale", *a)[0]

    assert call(w=None) == 1
    assert call(best=None) == 1
    assert call(g=96) == 2
    assert call(k=200) == 2
    assert call(m=0) == 2
    assert call(m=9000) == 2
    assert call(ng=0) == 2
    assert call(ng=65) == 2
    assert call(n=0) == 2
    assert call(w=MISALIGNED) == 3
    assert call(wsb=ws - 1) == 4
    assert call(ws=None) == 4
    assert call(ws=FAKE + 16) == 3


def test_fold_argument_errors(lib):
    assert _status(lib, "awq_fold_inv_scale", None, FAKE, 16, FAKE, None)[0] == 1
    assert _status(lib, "awq_fold_inv_scale", FAKE, None, 16, FAKE, None)[0] == 1
    assert _status(lib, "awq_fold_inv_scale", FAKE, FAKE, 16, None, None)[0] == 1
    assert _status(lib, "awq_fold_inv_scale", FAKE, FAKE, 0, FAKE, None)[0] == 2
    st, msg = _status(lib, "awq_fold_inv_scale", FAKE + 1, FAKE, 16, FAKE, None)
    assert st == 3 and "aligned" in msg


def test_fold_rows_argument_errors(lib):
    assert _status(lib, "awq_fold_inv_scale_rows", None, FAKE, 4, 16, FAKE, None)[0] == 1
    assert _status(lib, "awq_fold_inv_scale_rows", FAKE, FAKE, 0, 16, FAKE, None)[0] == 2
    assert _status(lib, "awq_fold_inv_scale_rows", FAKE, FAKE, 4, 0, FAKE, None)[0] == 2
    st, msg = _status(lib, "awq_fold_inv_scale_rows", FAKE, FAKE + 1, 4, 16, FAKE, None)
    assert st == 3 and "aligned" in msg


def test_pack_argument_errors(lib):
    base = [FAKE, None, 16, 256, 128, FAKE, FAKE, FAKE, None, None]

    def call(**kw):
        a = list(base)
        names = ["w", "s", "n", "k", "g", "qw", "sc", "qz", "bad", "st"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_pack_int4", *a)[0]

    assert call(w=None) == 1
    assert call(qz=None) == 1
    assert call(g=16) == 2
    assert call(k=192) == 2
    assert call(k=64) == 2
    assert call(n=0) == 2
    assert call(qw=MISALIGNED) == 3
    assert call(s=MISALIGNED) == 3


def test_linear_argument_errors(lib):
    base = [FAKE, FAKE, FAKE, FAKE, None, 1, 64, 256, 128, FAKE, None, 0, None]

    def call(**kw):
        a = list(base)
        names = ["x", "qw", "sc", "qz", "inv", "m", "n", "k", "g", "y", "ws", "wsb", "st"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_linear_w4a16", *a)[0]

    assert call(x=None) == 1
    assert call(y=None) == 1
    assert call(g=48) == 2
    assert call(k=96, g=32) == 2
    assert call(m=0) == 2
    assert call(n=0) == 2
    assert call(x=MISALIGNED) == 3
    assert call(qw=FAKE + 4) == 3
    # scales are read as 32-bit words of two groups
    assert call(sc=FAKE + 2) == 3
    # inv_s16 is read with 16-byte loads
    assert call(inv=FAKE + 2) == 3
    assert call(inv=FAKE + 8) == 3
    # 64 tokens run the prefill GEMM, which stages x * inv_s16 in the workspace
    need = lib.awq_linear_workspace_size(64, 64, 256, 128)
    assert need > 0
    assert call(m=64, ws=None) == 4
    assert call(m=64, ws=FAKE, wsb=need - 1) == 4
    assert call(m=64, ws=FAKE + 16, wsb=need) == 3


def test_linear_workspace_sizes(lib):
    """The size queries run the call's launch plan without launching (CPU only):
    no scratch for the decode GEMV and the fused skinny kernels, x_tilde slots
    and split-K partial tiles for the GEMM, 0 for invalid shapes."""
    C = __import__("ctypes")
    for m in (1, 2, 8, 16):
        for n, k in ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)):
            assert lib.awq_linear_workspace_size(m, n, k, 128) == 0, (m, n, k)
            assert lib.awq_linear_workspace_size(m, n, k, 64) == 0, (m, n, k)
    # m = 2048: one x_tilde slot of m * k halves per linear, no split
    assert lib.awq_linear_workspace_size(2048, 4096, 4096, 128) == 2048 * 4096 * 2
    assert lib.awq_linear_workspace_size(2048, 4096, 14336, 128) == 2048 * 14336 * 2
    ns = (C.c_int64 * 3)(4096, 1024, 1024)
    assert lib.awq_linear_group_workspace_size(ns, 3, 2048, 4096, 128) == 3 * 2048 * 4096 * 2
    assert lib.awq_linear_group_workspace_size(ns, 3, 1, 4096, 128) == 0
    # 33 tokens: 64-row tiles split along K, partial tiles after the x_tilde slot
    assert lib.awq_linear_workspace_size(33, 4096, 4096, 128) > 33 * 4096 * 2
    # 17-32 tokens: linears above 16 MiB of packed weights run the GEMM
    assert lib.awq_linear_workspace_size(32, 14336, 4096, 128) > 0
    assert lib.awq_linear_workspace_size(32, 4096, 4096, 128) == 0
    # invalid shapes
    assert lib.awq_linear_workspace_size(0, 64, 256, 128) == 0
    assert lib.awq_linear_workspace_size(64, 64, 96, 32) == 0
    assert lib.awq_linear_group_workspace_size(None, 1, 64, 256, 128) == 0
    assert lib.awq_linear_group_workspace_size(ns, 5, 64, 4096, 128) == 0
    # 3/8-bit: scratch only from 17 tokens (x * inv_s16, and partial tiles)
    assert lib.awq_linear_wbit_workspace_size(16, 14336, 4096, 128, 3, 1) == 0
    assert lib.awq_linear_wbit_workspace_size(2048, 4096, 4096, 128, 8, 1) == 2048 * 4096 * 2
    assert lib.awq_linear_wbit_workspace_size(2048, 4096, 4096, 128, 8, 0) == 0
    assert (lib.awq_linear_wbit_workspace_size(64, 4096, 4096, 128, 4, 1)
            == lib.awq_linear_workspace_size(64, 4096, 4096, 128))


def test_search_wbit_argument_errors(lib):
    ws = lib.awq_search_workspace_size(64, 256, 16, 128, 20)
    base = [FAKE, FAKE, FAKE, 64, 256, 16, 128, 20, 3, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    names = ["w", "x", "a", "n", "k", "m", "g", "ng", "wb", "best", "s", "inv", "loss", "ws", "wsb",
             "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_search_scale_wbit", *a)

    for wb in (0, 2, 5, 16):
        st, msg = call(wb=wb)
        assert st == 2 and "w_bit" in msg and msg.startswith("awq_search_scale_wbit"), msg
    assert call(w=None)[0] == 1
    assert call(g=96)[0] == 2
    assert call(m=9000)[0] == 2
    assert call(w=MISALIGNED)[0] == 3
    assert call(wsb=ws - 1)[0] == 4
    # the 4-bit entry keeps its own name in its messages
    st, msg = _status(lib, "awq_search_scale", FAKE, FAKE, FAKE, 64, 256, 16, 96, 20, FAKE, FAKE,
                      FAKE, FAKE, FAKE, ws, None)
    assert st == 2 and msg.startswith("awq_search_scale:"), msg


def test_pack_wbit_argument_errors(lib):
    base = [FAKE, None, 16, 256, 128, 8, FAKE, FAKE, FAKE, None, None]
    names = ["w", "s", "n", "k", "g", "wb", "qw", "sc", "qz", "bad", "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_pack_wbit", *a)

    for wb in (1, 2, 6, 7):
        st, msg = call(wb=wb)
        assert st == 2 and "w_bit" in msg, msg
    assert call(w=None)[0] == 1
    assert call(g=16)[0] == 2
    assert call(k=192)[0] == 2
    assert call(n=0)[0] == 2
    assert call(qw=MISALIGNED)[0] == 3
    assert call(qz=FAKE + 2)[0] == 3


def test_linear_wbit_argument_errors(lib):
    base = [FAKE, FAKE, FAKE, FAKE, None, 1, 64, 256, 128, 3, FAKE, None, 0, None]
    names = ["x", "qw", "sc", "qz", "inv", "m", "n", "k", "g", "wb", "y", "ws", "wsb", "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_linear_wbit", *a)

    for wb in (2, 5, 16):
        st, msg = call(wb=wb)
        assert st == 2 and "w_bit" in msg, msg
    for wb in (3, 8):
        assert call(wb=wb, x=None)[0] == 1
        assert call(wb=wb, g=48)[0] == 2
        assert call(wb=wb, k=96, g=32)[0] == 2
        assert call(wb=wb, m=0)[0] == 2
        assert call(wb=wb, n=0)[0] == 2
        assert call(wb=wb, x=MISALIGNED)[0] == 3
        assert call(wb=wb, inv=FAKE + 8)[0] == 3
        assert call(wb=wb, qw=FAKE + 4)[0] == 3
        assert call(wb=wb, qz=FAKE + 2)[0] == 3
    # w_bit 4 takes the 4-bit entry's checks (qweight 16-byte aligned there)
    st, msg = call(wb=4, qw=FAKE + 4)
    assert st == 3 and "awq_linear_w4a16" in msg, msg
    # from 17 tokens the tiled GEMM stages x * inv_s16 in the workspace
    assert call(wb=3, m=64, inv=FAKE)[0] == 4


def test_packed_shapes():
    import weight_only_int4_awq_amd as P
    assert P.packed_shapes(5, 4096, 128, 4) == ((5, 512), (5, 32), (5, 4))
    assert P.packed_shapes(5, 4096, 128, 8) == ((5, 1024), (5, 32), (5, 8))
    assert P.packed_shapes(5, 4096, 128, 3) == ((5, 384), (5, 32), (5, 4))
    assert P.packed_shapes(5, 4160, 64, 8) == ((5, 1040), (5, 65), (5, 17))


def test_linear_bf16_argument_errors(lib):
    base = [FAKE, FAKE, FAKE, FAKE, None, 1, 64, 256, 128, FAKE, None, 0, None]
    names = ["x", "qw", "sc", "qz", "inv", "m", "n", "k", "g", "y", "ws", "wsb", "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_linear_w4a16_bf16", *a)

    st, msg = call(x=None)
    assert st == 1 and msg.startswith("awq_linear_w4a16_bf16"), msg
    assert call(g=48)[0] == 2
    assert call(k=96, g=32)[0] == 2
    assert call(m=0)[0] == 2
    assert call(x=MISALIGNED)[0] == 3
    assert _status(lib, "awq_linear_w4a16_group_bf16", None, 1, 1, 256, 128, None, 0, None)[0] == 1
    st, msg = _status(lib, "awq_linear_w4a16_group_bf16", _items(2), 5, 1, 256, 128, None, 0, None)
    assert st == 2 and msg.startswith("awq_linear_w4a16_group_bf16"), msg


def test_mixed_argument_errors(lib):
    assert _status(lib, "awq_salient_channels", None, 64, 3, FAKE, None)[0] == 1
    assert _status(lib, "awq_salient_channels", FAKE, 64, 65, FAKE, None)[0] == 2
    assert _status(lib, "awq_salient_channels", FAKE, 4096, 1025, FAKE, None)[0] == 2
    assert _status(lib, "awq_salient_channels", FAKE, 64, -1, FAKE, None)[0] == 2
    assert _status(lib, "awq_salient_channels", FAKE + 4, 64, 3, FAKE, None)[0] == 3
    assert _status(lib, "awq_channel_mask", FAKE, 3, 64, None, None)[0] == 1
    assert _status(lib, "awq_channel_mask", FAKE, 65, 64, FAKE, None)[0] == 2
    assert _status(lib, "awq_gather_channels", FAKE, 0, 64, FAKE, 3, FAKE, None)[0] == 2
    assert _status(lib, "awq_gather_channels", FAKE, 8, 64, None, 3, FAKE, None)[0] == 1
    ws = lib.awq_mixed_loss_workspace_size(64, 256, 16, 128)
    assert ws > lib.awq_search_workspace_size(64, 256, 16, 128, 1)
    assert lib.awq_mixed_loss_workspace_size(64, 256, 16, 96) == 0
    base = [FAKE, FAKE, FAKE, 64, 256, 16, 128, FAKE, FAKE, ws, None]
    names = ["w", "x", "keep", "n", "k", "m", "g", "loss", "ws", "wsb", "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return _status(lib, "awq_mixed_loss", *a)[0]

    assert call(keep=None) == 1
    assert call(g=96) == 2
    assert call(m=9000) == 2
    assert call(x=MISALIGNED) == 3
    assert call(wsb=ws - 1) == 4
    lbase = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1, 64, 256, 128, FAKE, None, 0, None]
    lnames = ["x", "qw", "sc", "qz", "keep", "ws", "idx", "cnt", "m", "n", "k", "g", "y", "wk", "wkb",
              "st"]

    def lcall(**kw):
        a = list(lbase)
        for key, v in kw.items():
            a[lnames.index(key)] = v
        return _status(lib, "awq_linear_mixed", *a)

    assert lcall(keep=None)[0] == 1
    assert lcall(ws=None)[0] == 1
    assert lcall(cnt=257)[0] == 2
    st, msg = lcall(g=48)
    assert st == 2 and msg.startswith("awq_linear_mixed"), msg
    assert lcall(x=MISALIGNED)[0] == 3
    assert lcall(keep=FAKE + 2)[0] == 3          # keep16 is read as inv_s16: 16-byte loads
    assert lcall(m=64, cnt=0)[0] == 4            # the quantized part's GEMM needs the workspace


def test_python_binding_has_the_c_names():
    import weight_only_int4_awq_amd as P
    for name in ("awq_calib_stats", "awq_search_scale", "awq_search_workspace_size",
                 "awq_pack_int4", "awq_linear_w4a16", "awq_search_scale_wbit", "awq_pack_wbit",
                 "awq_linear_wbit", "awq_linear_w4a16_bf16", "awq_linear_w4a16_group_bf16",
                 "awq_salient_channels", "awq_channel_mask", "awq_gather_channels", "awq_mixed_loss",
                 "awq_linear_mixed"):
        assert callable(getattr(P, name))


def test_product_package_never_imports_the_oracle():
    pkg = ROOT / "weight_only_int4_awq_amd"
    for f in pkg.rglob("*"):
        if f.suffix in (".py", ".hip", ".h", ".cpp"):
            text = f.read_text()
            assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), f
            assert "awq_oracle" not in text, f


def _items(count, **over):
    from weight_only_int4_awq_amd import _lib
    arr = (_lib.LinearItem * max(count, 1))()
    for i in range(max(count, 1)):
        a = arr[i]
        a.x = a.qweight = a.scales = a.qzeros = a.y = FAKE
        a.inv_s16 = None
        a.n = 64
        for key, val in over.items():
            setattr(a, key, val)
    return arr


def test_linear_group_argument_errors(lib):
    def call(*a):
        return _status(lib, "awq_linear_w4a16_group", *a, None, 0, None)

    assert call(None, 1, 1, 256, 128)[0] == 1
    assert call(_items(1), 0, 1, 256, 128)[0] == 2
    assert call(_items(5), 5, 1, 256, 128)[0] == 2
    assert call(_items(2, y=None), 2, 1, 256, 128)[0] == 1
    assert call(_items(2, n=0), 2, 1, 256, 128)[0] == 2
    assert call(_items(2), 2, 1, 200, 128)[0] == 2
    assert call(_items(2), 2, 0, 256, 128)[0] == 2
    st, msg = call(_items(2, x=MISALIGNED), 2, 1, 256, 128)
    assert st == 3 and "awq_linear_w4a16_group" in msg
    assert call(_items(2, inv_s16=FAKE + 4), 2, 1, 256, 128)[0] == 3
    st, msg = call(_items(2), 2, 64, 256, 128)
    assert st == 4 and "workspace" in msg, msg
