"""ctypes loader for libmla_amd.so (the C ABI of include/mla.h).

Raises ``MlaLibraryError`` when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_amd.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mla.h")

MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(7)
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2


class MlaLibraryError(RuntimeError):
    pass


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        extra = f" (hipError {hip_error})" if status == MLA_ERR_HIP else ""
        super().__init__(f"{fn}: {msg}{extra}")


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("latent", ctypes.c_void_p),
        ("rope", ctypes.c_void_p),
        ("latent_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("latent_dtype", ctypes.c_int32),
        ("rope_dtype", ctypes.c_int32),
        ("latent_stride_b", ctypes.c_int64),
        ("latent_stride_tok", ctypes.c_int64),
        ("rope_stride_b", ctypes.c_int64),
        ("rope_stride_tok", ctypes.c_int64),
        ("scale_stride_b", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
    ]


_lib = None

_SIGS = {
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_hip_error": (ctypes.c_int, []),
    "mla_version": (ctypes.c_int, []),
    "mla_absorb_q": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "mla_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "mla_decode_auto_splits": (ctypes.c_int, [ctypes.c_int] * 3),
    "mla_decode_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(CacheDesc),
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "mla_decode_partial": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(CacheDesc),
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]),
    "mla_decode_partial_warm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.POINTER(CacheDesc), ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                               ctypes.c_void_p]),
    "mla_decode_combine": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "mla_decode_combine_uv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
    "mla_uv_out": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "mla_decode_attn_noalloc_max_bytes": (ctypes.c_size_t, []),
    "mla_decode_attn_noalloc_splits": (ctypes.c_int, [ctypes.c_int] * 4),
    "mla_decode_attn_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(CacheDesc),
                                               ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p]),
    "mla_decode_step_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "mla_decode_step_init": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_decode_step": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.POINTER(CacheDesc),
                                                                ctypes.c_void_p] + [ctypes.c_int] * 6
                        + [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 5),
    "mla_cache_append_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int]),
    "mla_proj_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "mla_query_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "mla_query_proj": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 6
                       + [ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_query_append_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 7),
    "mla_query_proj_append": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_void_p,
                                                                      ctypes.POINTER(CacheDesc)]
                              + [ctypes.c_int] * 7 + [ctypes.c_float] + [ctypes.c_void_p] * 4
                              + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_fold_q": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
                   + [ctypes.c_int] * 4 + [ctypes.c_void_p]),
    "mla_absorb_q_folded": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
                            + [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_out_proj": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
                     + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_fold_o": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
                   + [ctypes.c_int] * 4 + [ctypes.c_void_p]),
    "mla_mha_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "mla_mha_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "mla_cache_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.POINTER(CacheDesc), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """Load libmla_amd.so once; raise MlaLibraryError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MlaLibraryError(f"{LIB_PATH} not found: build it with "
                                  "`python -m mla_latent_kv_attn_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/mla.h."""
    with open(HEADER) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", txt)))


def check(fn: str, status: int) -> None:
    if status != MLA_OK:
        l = lib()
        raise MlaError(fn, status, l.mla_status_string(status).decode(), l.mla_last_hip_error())
