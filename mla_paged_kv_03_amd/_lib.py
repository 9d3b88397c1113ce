"""ctypes loader for libmla_decode.so (the gfx950 decode library)."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_DECODE_LIB selects another build of the same library (the tests use it
# for the host-sanitizer build); the default is the in-tree build.
LIB_PATH = os.environ.get("MLA_DECODE_LIB") or os.path.join(PKG, "libmla_decode.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mla_decode.h")

MLA_OK = 0
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL_ARG", -2: "MLA_ERR_BAD_SHAPE",
          -3: "MLA_ERR_UNSUPPORTED", -4: "MLA_ERR_WORKSPACE_TOO_SMALL", -5: "MLA_ERR_HIP",
          -6: "MLA_ERR_SCRATCH_LIMIT"}


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_workers", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
                ("max_split_slots", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("metadata_bytes", ctypes.c_size_t), ("num_splits_bytes", ctypes.c_size_t),
                ("workspace_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "mla_decode_plan": [_P, _I, _I, _I, _I, _I, _P, _P, ctypes.POINTER(PlanInfo), _P],
    "mla_decode_plan_fp8": [_P, _I, _I, _I, _P, _P, ctypes.POINTER(PlanInfo), _P],
    "mla_decode": [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                   ctypes.c_size_t, _P, _P, _P],
    "mla_decode_noalloc": [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P],
    "gqa_decode": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                   ctypes.c_size_t, _P, _P, _P],
    "attn_combine": [_P, _P, _P, _I, _I, _I, _P, _P, _P],
    "mla_kv_append": [_P, _P, _P, _P, _I, _I, _I, _I, _P],
    "gqa_kv_append": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P],
    "gqla_decode": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                    ctypes.c_size_t, _P, _P, _P],
    "gqla_absorb_query": [_P, _P, _P, _I, _I, _I, _P],
    "gqla_absorb_output": [_P, _P, _P, _I, _I, _I, _P],
    "gqla_expand_kv": [_P, _P, _P, _P, _P, ctypes.c_int64, _I, _P],
    "mla_decode_fp8": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                       ctypes.c_size_t, _P, _P, _P],
    "mla_kv_append_fp8": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P],
    "mla_kv_quantize_fp8": [_P, _P, _P, ctypes.c_int64, _P],
    "mla_decode_plan_host": [_P, _I, _I, _I, _I, _I, _I, _P, _P, ctypes.POINTER(PlanInfo)],
    "mla_check_pages": [_P, _P, _I, _I, _I, _P, _P],
    "mla_check_fp8_scales": [_P, ctypes.c_int64, _P, _P],
    "mla_status_string": [ctypes.c_int],
    "mla_ceiling_mfma": [_I, _I, _I, _I, _I, _P, _P],
    "mla_ceiling_stream_read": [_P, ctypes.c_size_t, _I, _P, _P],
    "mla_ceiling_lds_fill": [_P, ctypes.c_size_t, _I, _I, _P, _P],
    "mla_ceiling_lds_operand": [_I, _I, _I, _I, _P, _P],
    "mla_ceiling_block_write": [_P, ctypes.c_size_t, ctypes.c_size_t, _I, _P],
    "mla_profile_events": [_P, _P],
}

_lib = None


class DecodeError(RuntimeError):
    def __init__(self, fn, code):
        msg = _lib.mla_status_string(code).decode() if _lib is not None else ""
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({msg})")
        self.code = code


def lib():
    """Load the library; raise if it was not built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m mla_paged_kv_03_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "mla_status_string" else ctypes.c_int
        _lib = L
    return _lib


def check(fn: str, code: int) -> None:
    if code != MLA_OK:
        raise DecodeError(fn, code)


def header_functions() -> list[str]:
    """Names of the functions every header under include/ declares."""
    import glob
    names = []
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return names
