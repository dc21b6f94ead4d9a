"""ctypes binding of libulysses_sp.so: one Python function per C entry point,
same names, argument marshalling only.  Raises if the library is missing -
there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libulysses_sp.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ulysses_sp.h")

SP_OK = 0
SP_E_NULL = 1
SP_E_SHAPE = 2
SP_E_NOT_DIVISIBLE = 3
SP_E_ALIGN = 4
SP_E_RANK = 5
SP_E_WORKSPACE = 6
SP_E_HIP = 7
SP_E_DTYPE = 8
SP_E_SCRATCH = 9
SP_DTYPE_BF16 = 0
SP_DTYPE_F32 = 1

_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "sp_status_string": (ctypes.c_char_p, [_i]),
    "sp_abi_version": (_i, []),
    "ulysses_seq_to_head": (_i, [_vp, _vp, _i, _i64, _i, _i, _i, _i, _vp]),
    "ulysses_head_to_seq": (_i, [_vp, _vp, _i, _i64, _i, _i, _i, _i, _vp]),
    "ulysses_seq_to_head_kv": (_i, [_vp, _vp, _i, _i64, _i, _i, _i, _i, _vp]),
    "ulysses_head_to_seq_kv_grad": (_i, [_vp, _vp, _i, _i64, _i, _i, _i, _i, _i, _vp]),
    "sp_attn_workspace_bytes": (_sz, [_i64, _i, _i, _i]),
    "sp_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _i64, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "sp_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i, _i, _i, _f, _i, _vp, _vp,
                         _vp, _vp, _sz, _vp]),
    "sp_attn_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i, _i, _i, _f, _i,
                                 _vp, _vp, _vp, _vp]),
    "sp_attn_fwd_strided": (_i, [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i, _i, _i, _f, _vp, _i64,
                                 _vp, _vp, _sz, _vp]),
    "sp_attn_bwd_strided": (_i, [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64,
                                 _i, _i, _i, _f, _i, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz,
                                 _vp]),
    "sp_linear_ce_workspace_bytes": (_sz, [_i64, _i64]),
    "sp_linear_ce": (_i, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i, _vp, _vp, _vp, _vp,
                          _i64, _vp, _sz, _vp]),
    "sp_weighted_loss": (_i, [_vp, _vp, _i, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "sp_timing_enable": (_i, [_i]),
    "sp_timing_collect": (_i, [_vp, _i]),
}


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("min_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class SPError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/ulysses_sp.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m ulysses_sequence_parallelism_share_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sp_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != SP_OK:
        raise SPError(fn, status, status_string(status))


def call(name: str, *args) -> int:
    """Call a C entry point and return its raw status."""
    return getattr(lib(), name)(*args)
