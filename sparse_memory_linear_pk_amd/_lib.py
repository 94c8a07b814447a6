"""ctypes binding of libsdm.so (include/sdm.h).  Argument marshalling only: every
step of the layer runs in the library's HIP kernels.  There is no fallback: if
the library is not built, loading it raises."""
from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsdm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sdm.h")

SDM_OK, SDM_ERR_INVALID_ARG, SDM_ERR_UNSUPPORTED, SDM_ERR_OOM, SDM_ERR_DEVICE = range(5)
SDM_F32, SDM_BF16 = 0, 1


class SDMError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class Config(C.Structure):
    _fields_ = [("B", C.c_int), ("H", C.c_int), ("T", C.c_int), ("d", C.c_int), ("n_sub", C.c_int),
                ("dk", C.c_int), ("k", C.c_int), ("W", C.c_int), ("in_dtype", C.c_int), ("state_dtype", C.c_int),
                ("mem_stride", C.c_int)]


class Timing(C.Structure):
    _fields_ = [("ms_score", C.c_double), ("ms_select", C.c_double), ("ms_plan", C.c_double),
                ("ms_scan", C.c_double), ("n_score", C.c_longlong), ("n_select", C.c_longlong),
                ("n_plan", C.c_longlong), ("n_scan", C.c_longlong), ("ms_step", C.c_double),
                ("n_step", C.c_longlong), ("ms_train", C.c_double), ("ms_bwd_scan", C.c_double),
                ("ms_bwd_rows", C.c_double), ("ms_bwd_sub", C.c_double), ("n_train", C.c_longlong),
                ("n_bwd_scan", C.c_longlong), ("n_bwd_rows", C.c_longlong), ("n_bwd_sub", C.c_longlong),
                ("ms_project", C.c_double), ("n_project", C.c_longlong)]


def declared_symbols(header: str = HEADER) -> list[str]:
    """Names of the entry points include/sdm.h declares."""
    text = open(header).read()
    return re.findall(r"^SDM_API\s+[\w\s\*]+?\b(sdm_\w+)\s*\(", text, flags=re.M)


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_memory_linear_pk_amd.build` "
                           "or __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    vp, h = C.c_void_p, C.c_void_p
    sig = {
        "sdm_create": ([C.POINTER(Config), vp, C.POINTER(C.c_void_p)], C.c_int),
        "sdm_forward": ([h, vp, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_step": ([h, vp, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_step_static": ([C.POINTER(Config), vp, vp, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_forward_train": ([h, vp, vp, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_backward_workspace_bytes": ([C.POINTER(Config), C.POINTER(C.c_size_t)], C.c_int),
        "sdm_backward": ([h] + [vp] * 16, C.c_int),
        "sdm_project": ([h, C.c_int] + [vp] * 8, C.c_int),
        "sdm_broadcast_memory": ([h, vp, vp], C.c_int),
        "sdm_overlap": ([h, vp, vp, vp, vp, C.c_int, vp, vp, C.c_int, vp, vp], C.c_int),
        "sdm_destroy": ([h], C.c_int),
        "sdm_status_str": ([C.c_int], C.c_char_p),
        "sdm_last_error": ([], C.c_char_p),
        "sdm_workspace_bytes": ([C.POINTER(Config), C.POINTER(C.c_size_t)], C.c_int),
        "sdm_score": ([h, vp, vp, vp], C.c_int),
        "sdm_select": ([h, vp, vp, vp], C.c_int),
        "sdm_address": ([h, vp, vp, vp, vp], C.c_int),
        "sdm_address_pair": ([h, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_scan_with": ([h, vp, vp, vp, vp, vp, vp, vp, vp, vp], C.c_int),
        "sdm_set_timing": ([h, C.c_int], C.c_int),
        "sdm_get_timing": ([h, C.POINTER(Timing)], C.c_int),
        "sdm_pattern_probe": ([vp, C.c_int, C.c_long, C.c_int, C.c_int, C.c_int, C.c_uint, vp], C.c_int),
        "sdm_pattern_probe_mix": ([vp, C.c_int, C.c_long, C.c_int, C.c_long, C.c_int, C.c_int, C.c_int, C.c_int,
                                   C.c_uint, vp], C.c_int),
        "sdm_mem_stride_hint": ([C.POINTER(Config)], C.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def check(status: int, where: str):
    if status != SDM_OK:
        L = lib()
        raise SDMError(status, where, f"{L.sdm_status_str(status).decode()}: {L.sdm_last_error().decode()}")
