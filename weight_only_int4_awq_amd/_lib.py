"""ctypes handle on libawq_mi355x.so (the C ABI declared in include/awq_mi355x.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""
from __future__ import annotations

import ctypes as C
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libawq_mi355x.so"

STATUS = {0: "AWQ_OK", 1: "AWQ_ERR_NULL", 2: "AWQ_ERR_SHAPE", 3: "AWQ_ERR_ALIGN",
          4: "AWQ_ERR_WORKSPACE", 5: "AWQ_ERR_NONFINITE", 6: "AWQ_ERR_HIP", 7: "AWQ_ERR_UNSUPPORTED"}

# name -> (restype, argtypes)
SIGNATURES = {
    "awq_abi_version": (C.c_int32, []),
    "awq_last_error": (C.c_char_p, []),
    "awq_calib_stats": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]),
    "awq_search_workspace_size": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int64, C.c_int32, C.c_int32]),
    "awq_search_scale": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                   C.c_int64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "awq_pack_int4": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "awq_linear_workspace_size": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int64, C.c_int32]),
    "awq_linear_group_workspace_size": (C.c_size_t, [C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                                     C.c_int32]),
    "awq_linear_wbit_workspace_size": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int64, C.c_int32,
                                                    C.c_int32, C.c_int32]),
    "awq_linear_w4a16": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_int64, C.c_int64, C.c_int32, C.c_void_p,
                                   C.c_void_p, C.c_size_t, C.c_void_p]),
    "awq_fold_inv_scale": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "awq_fold_inv_scale_rows": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                                          C.c_void_p]),
    "awq_search_scale_wbit": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                        C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                        C.c_void_p]),
    "awq_pack_wbit": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "awq_linear_wbit": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_int64, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
}



class LinearItem(C.Structure):
    """awq_linear_item of the C header."""
    _fields_ = [("x", C.c_void_p), ("inv_s16", C.c_void_p), ("qweight", C.c_void_p),
                ("scales", C.c_void_p), ("qzeros", C.c_void_p), ("y", C.c_void_p),
                ("n", C.c_int64)]


SIGNATURES["awq_linear_w4a16_group"] = (C.c_int, [C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                                  C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p])
SIGNATURES["awq_linear_w4a16_bf16"] = SIGNATURES["awq_linear_w4a16"]
SIGNATURES["awq_salient_channels"] = (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p])
SIGNATURES["awq_channel_mask"] = (C.c_int, [C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p])
SIGNATURES["awq_gather_channels"] = (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32,
                                               C.c_void_p, C.c_void_p])
SIGNATURES["awq_mixed_loss_workspace_size"] = (C.c_size_t, [C.c_int64, C.c_int64, C.c_int64, C.c_int32])
SIGNATURES["awq_mixed_loss"] = (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                          C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t,
                                          C.c_void_p])
SIGNATURES["awq_linear_mixed"] = (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                            C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t,
                                            C.c_void_p])
SIGNATURES["awq_linear_w4a16_group_bf16"] = SIGNATURES["awq_linear_w4a16_group"]
SIGNATURES["awq_linear_noalloc_scratch_bytes"] = (C.c_size_t, [])
SIGNATURES["awq_linear_w4a16_group_noalloc"] = (C.c_int, [C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                                          C.c_int32, C.c_void_p])

_lib = None


class AWQError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


def load() -> C.CDLL:
    """Load the built library (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m weight_only_int4_awq_amd.build` "
            "(no CPU fallback exists for any step of the path)")
    lib = C.CDLL(str(LIB_PATH))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        msg = load().awq_last_error()
        raise AWQError(fn, status, msg.decode() if msg else "")
