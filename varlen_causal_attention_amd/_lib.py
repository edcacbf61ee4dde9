"""ctypes loader for libvca_attn.so: signatures and status handling only.

The library must have been built in-tree (``python -m
varlen_causal_attention_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# VCA_ATTN_LIB names another build of the same library (e.g. one with the host
# code built under AddressSanitizer for the host-side tests).
LIB_PATH = os.environ.get("VCA_ATTN_LIB") or os.path.join(HERE, "libvca_attn.so")

ATTN_OK = 0
ATTN_E_INVALID = -1
ATTN_E_UNSUPPORTED = -2
ATTN_E_WORKSPACE = -3
ATTN_E_HIP = -4
ATTN_BF16 = 0
ATTN_F32 = 1
ATTN_F16 = 2
ATTN_DQ_ACCUMULATE = 1
ATTN_ROWS_ASSIGN = 0
ATTN_ROWS_ASSIGN_ZERO_REST = 1
ATTN_ROWS_ADD = 2
ATTN_NOALLOC_MAX_ITEMS = 524256  # work-list entries the no-allocation forward's static scratch holds

EXPORTED = (
    "attn_last_error", "attn_version", "attn_is_supported", "attn_fwd_dense", "attn_fwd_varlen",
    "attn_fwd_varlen_noalloc",
    "attn_bwd_dense", "attn_bwd_varlen", "attn_merge", "attn_doc_segments", "attn_doc_cu_seqlens",
    "attn_dense_route",
    "attn_zero_rows", "attn_timing_enable", "attn_timing_read", "attn_ring_segments",
    "attn_ring_inplace_preferred", "attn_gather_rows", "attn_scatter_rows", "attn_gather_lse",
    "attn_scatter_lse", "attn_merge_rows", "attn_fwd_dense_ex", "attn_fwd_varlen_ex",
    "attn_bwd_dense_ex", "attn_bwd_varlen_ex",
)

_P = C.c_void_p
_I = C.c_int
_F = C.c_float
_I64P = C.POINTER(C.c_int64)
_SZP = C.POINTER(C.c_size_t)
_I32P = C.POINTER(C.c_int32)



class AttnExt(C.Structure):
    """struct attn_ext: left window (0 = none) and softcap (0 = none)."""
    _fields_ = [("window", C.c_int), ("softcap", C.c_float)]


_SIGS = {
    "attn_last_error": (C.c_char_p, []),
    "attn_version": (_I, []),
    "attn_is_supported": (_I, [_I, _I, _I]),
    "attn_fwd_dense": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I64P, _F, _I,
                            _P, _SZP, _P]),
    "attn_fwd_varlen": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                             _I64P, _F, _I, _P, _SZP, _P]),
    "attn_fwd_varlen_noalloc": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                     _I, _I, _I64P, _F, _I, _P]),
    "attn_bwd_dense": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                            _I64P, _F, _I, _I, _P, _SZP, _P]),
    "attn_bwd_varlen": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                             _I, _I, _I, _I, _I64P, _F, _I, _I, _P, _SZP, _P]),
    "attn_fwd_dense_ex": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I64P, _F, _I,
                               _P, _P, _SZP, _P]),
    "attn_fwd_varlen_ex": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                _I, _I64P, _F, _I, _P, _P, _SZP, _P]),
    "attn_bwd_dense_ex": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                               _I, _I64P, _F, _I, _P, _I, _P, _SZP, _P]),
    "attn_bwd_varlen_ex": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                _I, _I, _I, _I, _I, _I64P, _F, _I, _P, _I, _P, _SZP, _P]),
    "attn_merge": (_I, [_P, _I, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_doc_segments": (_I, [_I32P, _I, _I, _I, _I, _I, _I, _I, _I32P, _I32P, _I,
                               C.POINTER(C.c_int)]),
    "attn_doc_cu_seqlens": (_I, [_I32P, _I, _I, _I, _I, _I, _I, _I, _I32P, _I32P, _I,
                                 C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int)]),
    "attn_dense_route": (_I, [_I32P, _I, _I, _I, _I, _I, _I, _I, _P, C.POINTER(C.c_int)]),
    "attn_zero_rows": (_I, [_P, _I, C.c_int64, C.c_int64, C.c_int64, _P, C.c_int64, C.c_int64, _P,
                            _I, _I, _I, _I, _P]),
    "attn_ring_segments": (_I, [_I32P, _I, _I32P, _I, _I, _I32P, _I32P, _I32P, _I32P, _I,
                                C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int),
                                C.POINTER(C.c_int), C.POINTER(C.c_int)]),
    "attn_ring_inplace_preferred": (_I, [C.c_int64, C.c_int64, C.c_int64, _I, _I, _I]),
    "attn_gather_rows": (_I, [_I, _P, C.c_int64, C.c_int64, C.c_int64, _P, _I, _I, _I, _I, _I, _P,
                              _I, _P]),
    "attn_scatter_rows": (_I, [_I, _P, _P, _I, _I, _I, _P, C.c_int64, C.c_int64, C.c_int64, _I,
                               _I, _I, _P]),
    "attn_gather_lse": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "attn_scatter_lse": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _P]),
    "attn_merge_rows": (_I, [_P, C.c_int64, C.c_int64, C.c_int64, _P, _I, _I, _P, _I, _P, _P, _I,
                             _I, _I, _P]),
    "attn_timing_enable": (_I, [_I]),
    "attn_timing_read": (_I, [_I, C.c_char_p, _I, C.POINTER(C.c_float), C.POINTER(C.c_int)]),
}

_lib = None


class AttnError(RuntimeError):
    """A HIP runtime failure reported by the library."""


def load() -> C.CDLL:
    """Load the built library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m varlen_causal_attention_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, what: str) -> None:
    """Map a status code to an exception (ValueError for argument problems)."""
    if status == ATTN_OK:
        return
    msg = load().attn_last_error().decode()
    if status == ATTN_E_HIP:
        raise AttnError(f"{what}: {msg}")
    kind = {ATTN_E_INVALID: "invalid", ATTN_E_UNSUPPORTED: "unsupported",
            ATTN_E_WORKSPACE: "workspace"}.get(status, f"status {status}")
    raise ValueError(f"{what}: {kind}: {msg}")


def i64_array(values) -> C.Array:
    arr = (C.c_int64 * len(values))(*[int(x) for x in values])
    return arr
