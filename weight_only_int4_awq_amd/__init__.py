"""MI355X-native AWQ W4A16 hot path: Python binding of libawq_mi355x.so.

The functions below carry the names of the C entry points and only marshal
arguments: they check devices, dtypes, shapes and contiguity, allocate outputs
with torch (device memory plumbing) and pass raw device pointers plus
``torch.cuda.current_stream()`` to the library.  Every step of the path runs in
the library's HIP kernels; there is no fallback.

    awq_calib_stats(x)                          -> mean_abs  float64 [k]
    awq_search_scale(w, x, mean_abs, g, n_grid) -> (best_idx int32 [1], s16, inv_s16, losses)
    awq_pack_int4(w, s16, g)                    -> (qweight, scales, qzeros, nonfinite int32 [1])
    awq_linear_w4a16(x, qweight, scales, qzeros, inv_s16, g) -> y fp16 [m, n]
    awq_linear_w4a16_group([(x, qweight, scales, qzeros, inv_s16, out), ...], g) -> [y, ...]

The linear calls take an optional ``workspace`` (a uint8 device tensor of at
least the size the library's query returns); without one the binding
allocates it with torch for the call.  The library itself allocates nothing.
"""
from __future__ import annotations

from . import _lib
from ._lib import AWQError  # noqa: F401

__all__ = ["awq_calib_stats", "awq_search_workspace_size", "awq_search_scale", "awq_fold_inv_scale",
           "awq_linear_workspace_size", "awq_linear_group_workspace_size", "awq_linear_wbit_workspace_size",
           "awq_pack_int4", "awq_linear_w4a16", "awq_linear_w4a16_group",
           "awq_search_scale_wbit", "awq_pack_wbit", "awq_linear_wbit", "packed_shapes",
           "awq_linear_w4a16_bf16", "awq_linear_w4a16_group_bf16",
           "awq_salient_channels", "awq_channel_mask", "awq_gather_channels", "awq_mixed_loss",
           "awq_linear_mixed", "awq_fold_inv_scale_rows", "awq_linear_w4a16_group_noalloc",
           "AWQError", "load"]


def load():
    return _lib.load()


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _out_tensor(t, dtype, shape, name):
    _dev_tensor(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _dev_tensor(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")
    return t


def _workspace(need, device, workspace):
    """(pointer, bytes) of the call's workspace: the caller's uint8 tensor, or
    one allocated with torch when none is given (None when need is 0)."""
    torch = _torch()
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _dev_tensor(workspace, torch.uint8, "workspace")
    return workspace.data_ptr(), workspace.numel()


def awq_linear_workspace_size(m, n, k, g=128):
    """Device scratch bytes awq_linear_w4a16 (and its bf16 and mixed forms)
    needs for this shape (0 for the decode GEMV and the fused skinny kernels)."""
    return int(_lib.load().awq_linear_workspace_size(m, n, k, g))


def awq_linear_group_workspace_size(ns, m, k, g=128):
    """Device scratch bytes of awq_linear_w4a16_group for linears of widths ns."""
    import ctypes as C
    arr = (C.c_int64 * len(ns))(*ns)
    return int(_lib.load().awq_linear_group_workspace_size(arr, len(ns), m, k, g))


def awq_linear_wbit_workspace_size(m, n, k, g=128, w_bit=4, has_inv_s16=True):
    return int(_lib.load().awq_linear_wbit_workspace_size(m, n, k, g, w_bit, 1 if has_inv_s16 else 0))


def awq_calib_stats(x, out=None):
    """Per-channel mean |x| over tokens: x fp16 [m, k] -> float64 [k]."""
    torch = _torch()
    _dev_tensor(x, torch.float16, "x", 2)
    m, k = x.shape
    if out is None:
        out = torch.empty(k, dtype=torch.float64, device=x.device)
    _out_tensor(out, torch.float64, (k,), "out")
    _lib.check("awq_calib_stats", _lib.load().awq_calib_stats(_ptr(x), m, k, _ptr(out), _stream()))
    return out


def awq_search_workspace_size(n, k, m, g=128, n_grid=20):
    return int(_lib.load().awq_search_workspace_size(n, k, m, g, n_grid))


def awq_search_scale(w, x, mean_abs, g=128, n_grid=20, workspace=None, out=None):
    """Grid search of s = mean_abs ** alpha.  Returns (best_idx int32 [1], s16 fp16 [k],
    inv_s16 fp16 [k], losses float64 [n_grid]) as device tensors (written into
    ``out`` when given)."""
    return _search(w, x, mean_abs, g, n_grid, None, workspace, out)


def awq_search_scale_wbit(w, x, mean_abs, g=128, n_grid=20, w_bit=4, workspace=None, out=None):
    """awq_search_scale for codes of w_bit = 3, 4 or 8 bits."""
    return _search(w, x, mean_abs, g, n_grid, w_bit, workspace, out)


def _search(w, x, mean_abs, g, n_grid, w_bit, workspace, out):
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    _dev_tensor(x, torch.float16, "x", 2)
    _dev_tensor(mean_abs, torch.float64, "mean_abs", 1)
    n, k = w.shape
    m = x.shape[0]
    if x.shape[1] != k or mean_abs.shape[0] != k:
        raise ValueError("w, x and mean_abs disagree on k")
    need = awq_search_workspace_size(n, k, m, g, n_grid)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    dev = w.device
    if out is None:
        best = torch.empty(1, dtype=torch.int32, device=dev)
        s16 = torch.empty(k, dtype=torch.float16, device=dev)
        inv = torch.empty(k, dtype=torch.float16, device=dev)
        losses = torch.empty(n_grid, dtype=torch.float64, device=dev)
    else:
        best, s16, inv, losses = out
    _out_tensor(best, torch.int32, (1,), "best_idx")
    _out_tensor(s16, torch.float16, (k,), "s16")
    _out_tensor(inv, torch.float16, (k,), "inv_s16")
    _out_tensor(losses, torch.float64, (n_grid,), "losses")
    _dev_tensor(workspace, torch.uint8, "workspace")
    if w_bit is None:
        st = _lib.load().awq_search_scale(_ptr(w), _ptr(x), _ptr(mean_abs), n, k, m, g, n_grid,
                                          _ptr(best), _ptr(s16), _ptr(inv), _ptr(losses),
                                          _ptr(workspace), workspace.numel(), _stream())
        _lib.check("awq_search_scale", st)
    else:
        st = _lib.load().awq_search_scale_wbit(_ptr(w), _ptr(x), _ptr(mean_abs), n, k, m, g,
                                               n_grid, w_bit, _ptr(best), _ptr(s16), _ptr(inv),
                                               _ptr(losses), _ptr(workspace), workspace.numel(),
                                               _stream())
        _lib.check("awq_search_scale_wbit", st)
    return best, s16, inv, losses


def awq_fold_inv_scale(v, s16, out=None):
    """fp16_rn(v / s16) per channel (fp16 [k] each): the weight of the
    operation producing a linear's input with the linear's 1/s folded in, so
    the linear runs with inv_s16=None.  Returns the fp16 [k] tensor."""
    torch = _torch()
    _dev_tensor(v, torch.float16, "v", 1)
    _dev_tensor(s16, torch.float16, "s16", 1)
    k = v.shape[0]
    if s16.shape[0] != k:
        raise ValueError("v and s16 must have the same length")
    if out is None:
        out = torch.empty(k, dtype=torch.float16, device=v.device)
    _out_tensor(out, torch.float16, (k,), "out")
    st = _lib.load().awq_fold_inv_scale(_ptr(v), _ptr(s16), k, _ptr(out), _stream())
    _lib.check("awq_fold_inv_scale", st)
    return out


def awq_fold_inv_scale_rows(w, s16, out=None):
    """fp16_rn(w[j, :] / s16[j]) (w fp16 [n, k], s16 fp16 [n]): the weight of the
    linear producing another linear's input with that linear's 1/s folded
    into its output rows.  Returns the fp16 [n, k] tensor."""
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    _dev_tensor(s16, torch.float16, "s16", 1)
    n, k = w.shape
    if s16.shape[0] != n:
        raise ValueError("s16 must have one entry per row of w")
    o = out if out is not None else torch.empty((n, k), dtype=torch.float16, device=w.device)
    _out_tensor(o, torch.float16, (n, k), "out")
    st = _lib.load().awq_fold_inv_scale_rows(_ptr(w), _ptr(s16), n, k, _ptr(o), _stream())
    _lib.check("awq_fold_inv_scale_rows", st)
    return o


def awq_pack_int4(w, s16=None, g=128, out=None):
    """Quantize and pack w (fp16 [n, k]) at channel scale s16 (fp16 [k] or None).
    Returns (qweight int32 [n, k/8], scales fp16 [n, k/g], qzeros int32
    [n, ceil(k/(8g))], nonfinite int32 [1]); the packed words are uint32 bit
    patterns held in int32 tensors."""
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    n, k = w.shape
    if s16 is not None:
        _dev_tensor(s16, torch.float16, "s16", 1)
        if s16.shape[0] != k:
            raise ValueError("s16 must have k entries")
    dev = w.device
    if out is None:
        qw = torch.empty((n, k // 8), dtype=torch.int32, device=dev)
        sc = torch.empty((n, k // g), dtype=torch.float16, device=dev)
        qz = torch.empty((n, -(-k // (8 * g))), dtype=torch.int32, device=dev)
        bad = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        qw, sc, qz, bad = out
    _out_tensor(qw, torch.int32, (n, k // 8), "qweight")
    _out_tensor(sc, torch.float16, (n, k // g), "scales")
    _out_tensor(qz, torch.int32, (n, -(-k // (8 * g))), "qzeros")
    if bad is not None:
        _out_tensor(bad, torch.int32, (1,), "nonfinite")
    st = _lib.load().awq_pack_int4(_ptr(w), _ptr(s16), n, k, g, _ptr(qw), _ptr(sc), _ptr(qz),
                                   _ptr(bad), _stream())
    _lib.check("awq_pack_int4", st)
    return qw, sc, qz, bad


def packed_shapes(n, k, g, w_bit=4):
    """(qweight, scales, qzeros) shapes of the packed layout for w_bit bits."""
    if w_bit == 4:
        return (n, k // 8), (n, k // g), (n, -(-k // (8 * g)))
    if w_bit == 8:
        return (n, k // 4), (n, k // g), (n, -(-k // (4 * g)))
    if w_bit == 3:
        return (n, 3 * k // 32), (n, k // g), (n, -(-k // (8 * g)))
    raise ValueError("w_bit must be 3, 4 or 8")


def awq_pack_wbit(w, s16=None, g=128, w_bit=4, out=None):
    """awq_pack_int4 for codes of w_bit = 3, 4 or 8 bits (layouts of the C
    header).  Returns (qweight int32, scales fp16 [n, k/g], qzeros int32,
    nonfinite int32 [1])."""
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    n, k = w.shape
    if s16 is not None:
        _dev_tensor(s16, torch.float16, "s16", 1)
        if s16.shape[0] != k:
            raise ValueError("s16 must have k entries")
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    shq, shs, shz = packed_shapes(n, k, g, w_bit)
    dev = w.device
    if out is None:
        qw = torch.empty(shq, dtype=torch.int32, device=dev)
        sc = torch.empty(shs, dtype=torch.float16, device=dev)
        qz = torch.empty(shz, dtype=torch.int32, device=dev)
        bad = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        qw, sc, qz, bad = out
    _out_tensor(qw, torch.int32, shq, "qweight")
    _out_tensor(sc, torch.float16, shs, "scales")
    _out_tensor(qz, torch.int32, shz, "qzeros")
    if bad is not None:
        _out_tensor(bad, torch.int32, (1,), "nonfinite")
    st = _lib.load().awq_pack_wbit(_ptr(w), _ptr(s16), n, k, g, w_bit, _ptr(qw), _ptr(sc),
                                   _ptr(qz), _ptr(bad), _stream())
    _lib.check("awq_pack_wbit", st)
    return qw, sc, qz, bad


def awq_linear_wbit(x, qweight, scales, qzeros, inv_s16=None, g=128, w_bit=4, out=None, workspace=None):
    """awq_linear_w4a16 for the layouts of awq_pack_wbit: x fp16 [m, k] -> y fp16 [m, n]."""
    torch = _torch()
    _dev_tensor(x, torch.float16, "x", 2)
    _dev_tensor(qweight, torch.int32, "qweight", 2)
    _dev_tensor(scales, torch.float16, "scales", 2)
    _dev_tensor(qzeros, torch.int32, "qzeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    shq, shs, shz = packed_shapes(n, k, g, w_bit)
    if tuple(qweight.shape) != shq or tuple(scales.shape) != shs or tuple(qzeros.shape) != shz:
        raise ValueError("packed tensors do not match x, g and w_bit")
    if inv_s16 is not None:
        _dev_tensor(inv_s16, torch.float16, "inv_s16", 1)
        if inv_s16.shape[0] != k:
            raise ValueError("inv_s16 must have k entries")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float16, device=x.device)
    _out_tensor(y, torch.float16, (m, n), "y")
    wp, wb = _workspace(awq_linear_wbit_workspace_size(m, n, k, g, w_bit, inv_s16 is not None), x.device,
                        workspace)
    st = _lib.load().awq_linear_wbit(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros),
                                     _ptr(inv_s16), m, n, k, g, w_bit, _ptr(y), wp, wb, _stream())
    _lib.check("awq_linear_wbit", st)
    return y


def awq_linear_w4a16(x, qweight, scales, qzeros, inv_s16=None, g=128, out=None, workspace=None):
    """y = (x * inv_s16) @ dequant(W)^T in fp16: x fp16 [m, k] -> y fp16 [m, n]."""
    return _linear(x, qweight, scales, qzeros, inv_s16, g, out, False, workspace)


def awq_linear_w4a16_bf16(x, qweight, scales, qzeros, inv_s16=None, g=128, out=None, workspace=None):
    """awq_linear_w4a16 with bf16 activations: x bf16 [m, k] -> y bf16 [m, n]
    (inv_s16 and the packed tensors as for fp16)."""
    return _linear(x, qweight, scales, qzeros, inv_s16, g, out, True, workspace)


def _linear(x, qweight, scales, qzeros, inv_s16, g, out, bf, workspace):
    torch = _torch()
    adt = torch.bfloat16 if bf else torch.float16
    _dev_tensor(x, adt, "x", 2)
    _dev_tensor(qweight, torch.int32, "qweight", 2)
    _dev_tensor(scales, torch.float16, "scales", 2)
    _dev_tensor(qzeros, torch.int32, "qzeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if qweight.shape[1] * 8 != k or scales.shape != (n, k // g) or qzeros.shape != (n, -(-k // (8 * g))):
        raise ValueError("packed tensors do not match x and g")
    if inv_s16 is not None:
        _dev_tensor(inv_s16, torch.float16, "inv_s16", 1)
        if inv_s16.shape[0] != k:
            raise ValueError("inv_s16 must have k entries")
    y = out if out is not None else torch.empty((m, n), dtype=adt, device=x.device)
    _out_tensor(y, adt, (m, n), "y")
    fn = "awq_linear_w4a16_bf16" if bf else "awq_linear_w4a16"
    wp, wb = _workspace(awq_linear_workspace_size(m, n, k, g), x.device, workspace)
    st = getattr(_lib.load(), fn)(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros),
                                  _ptr(inv_s16), m, n, k, g, _ptr(y), wp, wb, _stream())
    _lib.check(fn, st)
    return y


def awq_linear_w4a16_group(items, g=128, workspace=None):
    """Independent linears with the same m and k (q, k, v of a layer; gate and
    up) in one call.  ``items`` holds up to four tuples (x, qweight, scales,
    qzeros, inv_s16, out) with x fp16 [m, k] and out fp16 [m, n] or None.
    Returns the list of outputs; each equals awq_linear_w4a16 of that linear."""
    return _linear_group(items, g, False, workspace)


def awq_linear_w4a16_group_bf16(items, g=128, workspace=None):
    """awq_linear_w4a16_group with bf16 activations (x and out bf16)."""
    return _linear_group(items, g, True, workspace)


def _linear_group(items, g, bf, workspace):
    torch = _torch()
    adt = torch.bfloat16 if bf else torch.float16
    if not 1 <= len(items) <= 4:
        raise ValueError("a group holds 1 to 4 linears")
    arr = (_lib.LinearItem * len(items))()
    outs = []
    m = k = None
    for i, (x, qweight, scales, qzeros, inv_s16, out) in enumerate(items):
        _dev_tensor(x, adt, "x", 2)
        _dev_tensor(qweight, torch.int32, "qweight", 2)
        _dev_tensor(scales, torch.float16, "scales", 2)
        _dev_tensor(qzeros, torch.int32, "qzeros", 2)
        mi, ki = x.shape
        if m is None:
            m, k = mi, ki
        elif (mi, ki) != (m, k):
            raise ValueError("the linears of a group must share m and k")
        n = qweight.shape[0]
        if qweight.shape[1] * 8 != k or scales.shape != (n, k // g) or qzeros.shape != (n, -(-k // (8 * g))):
            raise ValueError(f"linear {i}: packed tensors do not match x and g")
        if inv_s16 is not None:
            _dev_tensor(inv_s16, torch.float16, "inv_s16", 1)
            if inv_s16.shape[0] != k:
                raise ValueError(f"linear {i}: inv_s16 must have k entries")
        y = out if out is not None else torch.empty((m, n), dtype=adt, device=x.device)
        _out_tensor(y, adt, (m, n), "y")
        a = arr[i]
        a.x, a.inv_s16, a.qweight = _ptr(x), _ptr(inv_s16), _ptr(qweight)
        a.scales, a.qzeros, a.y, a.n = _ptr(scales), _ptr(qzeros), _ptr(y), n
        outs.append(y)
    fn = "awq_linear_w4a16_group_bf16" if bf else "awq_linear_w4a16_group"
    wp, wb = _workspace(awq_linear_group_workspace_size([int(a.n) for a in arr], m, k, g), outs[0].device,
                        workspace)
    st = getattr(_lib.load(), fn)(arr, len(items), m, k, g, wp, wb, _stream())
    _lib.check(fn, st)
    return outs


def awq_linear_w4a16_group_noalloc(items, g=128):
    """awq_linear_w4a16_group without a workspace: the library's static device
    scratch (awq_linear_noalloc_scratch_bytes() per GPU) serves the call, and
    nothing is allocated by the library or here (the outputs must be given).
    Calls that overlap on one GPU share that scratch and must be serialised."""
    torch = _torch()
    if not 1 <= len(items) <= 4:
        raise ValueError("a group holds 1 to 4 linears")
    arr = (_lib.LinearItem * len(items))()
    m = k = None
    for i, (x, qweight, scales, qzeros, inv_s16, out) in enumerate(items):
        _dev_tensor(x, torch.float16, "x", 2)
        if out is None:
            raise ValueError("the no-allocation call needs every output given")
        mi, ki = x.shape
        if m is None:
            m, k = mi, ki
        elif (mi, ki) != (m, k):
            raise ValueError("the linears of a group must share m and k")
        n = qweight.shape[0]
        _out_tensor(out, torch.float16, (m, n), "y")
        a = arr[i]
        a.x, a.inv_s16, a.qweight = _ptr(x), _ptr(inv_s16), _ptr(qweight)
        a.scales, a.qzeros, a.y, a.n = _ptr(scales), _ptr(qzeros), _ptr(out), n
    st = _lib.load().awq_linear_w4a16_group_noalloc(arr, len(items), m, k, g, _stream())
    _lib.check("awq_linear_w4a16_group_noalloc", st)
    return [it[5] for it in items]


# ---------------------------------------------------------------- mixed-precision baseline

def awq_salient_channels(mean_abs, count):
    """Indices (int32, ascending) of the ``count`` channels with the largest
    mean |x| (float64 [k] device tensor), ties to the lower index."""
    torch = _torch()
    _dev_tensor(mean_abs, torch.float64, "mean_abs", 1)
    k = mean_abs.shape[0]
    idx = torch.empty(max(count, 0), dtype=torch.int32, device=mean_abs.device)
    st = _lib.load().awq_salient_channels(_ptr(mean_abs), k, count, _ptr(idx) if count > 0 else None,
                                          _stream())
    _lib.check("awq_salient_channels", st)
    return idx


def awq_channel_mask(idx, k, out=None):
    """fp16 [k]: 1.0, and 0.0 on the channels idx (int32 device tensor)."""
    torch = _torch()
    _dev_tensor(idx, torch.int32, "idx", 1)
    keep = out if out is not None else torch.empty(k, dtype=torch.float16, device=idx.device)
    _out_tensor(keep, torch.float16, (k,), "keep16")
    cnt = idx.shape[0]
    st = _lib.load().awq_channel_mask(_ptr(idx) if cnt > 0 else None, cnt, k, _ptr(keep), _stream())
    _lib.check("awq_channel_mask", st)
    return keep


def awq_gather_channels(w, idx, out=None):
    """fp16 [count, n]: the columns idx of w (fp16 [n, k]), channel-major."""
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    _dev_tensor(idx, torch.int32, "idx", 1)
    n, k = w.shape
    cnt = idx.shape[0]
    ws = out if out is not None else torch.empty((cnt, n), dtype=torch.float16, device=w.device)
    _out_tensor(ws, torch.float16, (cnt, n), "w_s")
    st = _lib.load().awq_gather_channels(_ptr(w), n, k, _ptr(idx) if cnt > 0 else None, cnt,
                                         _ptr(ws) if cnt > 0 else None, _stream())
    _lib.check("awq_gather_channels", st)
    return ws


def awq_mixed_loss(w, x, keep16, g=128, workspace=None, out=None):
    """Output-error loss (float64 [1]) of the mixed-precision weight: RTN of w
    with the channels where keep16 is 0 kept in fp16."""
    torch = _torch()
    _dev_tensor(w, torch.float16, "w", 2)
    _dev_tensor(x, torch.float16, "x", 2)
    _dev_tensor(keep16, torch.float16, "keep16", 1)
    n, k = w.shape
    m = x.shape[0]
    if x.shape[1] != k or keep16.shape[0] != k:
        raise ValueError("w, x and keep16 disagree on k")
    lib = _lib.load()
    need = lib.awq_mixed_loss_workspace_size(n, k, m, g)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    loss = out if out is not None else torch.empty(1, dtype=torch.float64, device=w.device)
    _out_tensor(loss, torch.float64, (1,), "loss")
    st = lib.awq_mixed_loss(_ptr(w), _ptr(x), _ptr(keep16), n, k, m, g, _ptr(loss), _ptr(workspace),
                            workspace.numel(), _stream())
    _lib.check("awq_mixed_loss", st)
    return loss


def awq_linear_mixed(x, qweight, scales, qzeros, keep16, w_s, idx, g=128, out=None, workspace=None):
    """y = x Wm^T (fp16 [m, n]) for the RTN pack of W with the channels idx kept
    in fp16 (w_s [count, n], keep16 the matching mask)."""
    torch = _torch()
    _dev_tensor(x, torch.float16, "x", 2)
    _dev_tensor(qweight, torch.int32, "qweight", 2)
    _dev_tensor(scales, torch.float16, "scales", 2)
    _dev_tensor(qzeros, torch.int32, "qzeros", 2)
    _dev_tensor(keep16, torch.float16, "keep16", 1)
    _dev_tensor(idx, torch.int32, "idx", 1)
    m, k = x.shape
    n = qweight.shape[0]
    cnt = idx.shape[0]
    if cnt > 0:
        _dev_tensor(w_s, torch.float16, "w_s", 2)
        if tuple(w_s.shape) != (cnt, n):
            raise ValueError("w_s must be [count, n]")
    if qweight.shape[1] * 8 != k or keep16.shape[0] != k:
        raise ValueError("packed tensors or keep16 do not match x")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float16, device=x.device)
    _out_tensor(y, torch.float16, (m, n), "y")
    wp, wb = _workspace(awq_linear_workspace_size(m, n, k, g), x.device, workspace)
    st = _lib.load().awq_linear_mixed(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(keep16),
                                      _ptr(w_s) if cnt > 0 else None, _ptr(idx) if cnt > 0 else None,
                                      cnt, m, n, k, g, _ptr(y), wp, wb, _stream())
    _lib.check("awq_linear_mixed", st)
    return y

