"""ctypes declarations of the C ABI in include/swa.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

# SWA_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("SWA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

SWA_OK = 0
STATUS = {0: "SWA_OK", -1: "SWA_EINVAL", -2: "SWA_ENULL", -3: "SWA_EALIGN", -4: "SWA_EUNSUPPORTED",
          -5: "SWA_EWORKSPACE", -6: "SWA_EHIP"}
KIND = {"bf16": 0, "fp32": 1, "int8": 2, "int8_dither": 3}
LAYOUT = {"ring": 0, "paged": 1}

# Every symbol include/swa.h declares.
EXPORTS = ("swa_cache_reset", "kv_append", "decode_attn", "decode_attn_int8_witness",
           "decode_attn_int8_witness_tv", "decode_attn_int8_dither", "decode_step", "decode_step_int8",
           "decode_step_int8_static", "kv_truncate", "swa_workspace_bytes", "swa_workspace_init", "swa_validate",
           "swa_status_string")


class SwaCacheDesc(ctypes.Structure):
    """Mirror of ``swa_cache``."""

    _fields_ = [
        ("kind", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("W", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("pos", ctypes.c_void_p), ("next_position", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("witness", ctypes.c_void_p),
        ("k_stage", ctypes.c_void_p), ("v_stage", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
        ("request_id", ctypes.c_void_p), ("layer", ctypes.c_uint32),
        ("step_sync", ctypes.c_void_p),
    ]


class SwaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libswa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sliding_window_attention_ring_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, I32, SZ = ctypes.POINTER(SwaCacheDesc), ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "swa_cache_reset": (ctypes.c_int, [P, VP]),
            "kv_append": (ctypes.c_int, [P, VP, VP, I32, VP]),
            "decode_attn": (ctypes.c_int, [P, VP, VP, VP, SZ, VP]),
            "decode_attn_int8_witness": (ctypes.c_int, [P, VP, VP, VP, VP, VP, SZ, VP]),
            "decode_attn_int8_witness_tv": (ctypes.c_int, [P, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP, SZ,
                                                           VP]),
            "decode_attn_int8_dither": (ctypes.c_int, [P, VP, VP, VP, VP, VP, ctypes.c_float, ctypes.c_float, VP,
                                                       SZ, VP]),
            "decode_step": (ctypes.c_int, [P, VP, VP, VP, VP, VP, SZ, VP]),
            "decode_step_int8": (ctypes.c_int, [P, VP, VP, VP, VP, VP, VP, VP, ctypes.c_float, ctypes.c_float, VP,
                                                SZ, VP]),
            "decode_step_int8_static": (ctypes.c_int, [P, VP, VP, VP, VP, VP, VP, VP, ctypes.c_float,
                                                       ctypes.c_float, VP]),
            "kv_truncate": (ctypes.c_int, [P, VP, VP, VP]),
            "swa_workspace_bytes": (SZ, [P]),
            "swa_workspace_init": (ctypes.c_int, [VP, SZ, VP]),
            "swa_validate": (ctypes.c_int, [P, VP, VP]),
            "swa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().swa_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != SWA_OK:
        raise SwaError(status, what)
