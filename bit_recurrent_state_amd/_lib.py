"""Loads libqstate.so and declares the C ABI of include/qstate.h for ctypes.

There is no fallback: if the library is missing or does not load, this
raises, and nothing in the package computes the step any other way."""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqstate.so")

QSTATE_OK = 0
QSTATE_E_INVALID = -1
QSTATE_E_UNSUPPORTED = -2
QSTATE_E_LAUNCH = -3
QSTATE_E_NOMEM = -4

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2
VALUE_AXIS, KEY_AXIS = 0, 1

EXPORTS = (
    "qstate_state_bytes", "qstate_create", "qstate_load_fp32", "qstate_step",
    "qstate_readout", "qstate_store_fp32", "qstate_get_step", "qstate_set_step",
    "qstate_destroy", "qstate_strerror", "qstate_bits_by_decay",
)
# include/qstate_ceiling.h: bandwidth-ceiling kernels (measurement support)
CEILING_EXPORTS = ("qstate_ceiling_copy", "qstate_ceiling_rmw")


class QStateConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32), ("group", ctypes.c_int32), ("mixer", ctypes.c_int32),
        ("rounding", ctypes.c_int32), ("fp32_state", ctypes.c_int32),
        ("head_bits", ctypes.POINTER(ctypes.c_uint8)), ("seed", ctypes.c_uint64),
        ("layer", ctypes.c_uint32), ("group_axis", ctypes.c_int32),
        ("channel_bits", ctypes.POINTER(ctypes.c_uint8)), ("window", ctypes.c_int32),
        ("window_merge", ctypes.c_int32), ("lrb_threshold", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run "
                          "python -m bit_recurrent_state_amd.build")
    from . import build
    if all(os.path.exists(f) for f in build.SOURCES + build.HEADERS) and build.stale():
        raise ImportError(f"{LIB_PATH} was built from other sources or flags than those in "
                          "the package: run python -m bit_recurrent_state_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, c_int, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    cfgp = ctypes.POINTER(QStateConfig)
    sigs = {
        "qstate_state_bytes": (c_int, [cfgp, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "qstate_create": (c_int, [cfgp, P, P, ctypes.POINTER(P)]),
        "qstate_load_fp32": (c_int, [P, P, P]),
        "qstate_step": (c_int, [P, P, P, P, P, P, P, P]),
        "qstate_readout": (c_int, [P, P, P, P]),
        "qstate_store_fp32": (c_int, [P, P, P]),
        "qstate_get_step": (c_int, [P, ctypes.POINTER(ctypes.c_uint64)]),
        "qstate_set_step": (c_int, [P, ctypes.c_uint64]),
        "qstate_destroy": (c_int, [P]),
        "qstate_strerror": (ctypes.c_char_p, [c_int]),
        "qstate_bits_by_decay": (c_int, [P, c_int, c_int, ctypes.c_float, ctypes.c_uint8,
                                         ctypes.c_uint8, P]),
        "qstate_ceiling_copy": (c_int, [P, P, sz, c_int, P]),
        "qstate_ceiling_rmw": (c_int, [P, sz, ctypes.c_uint32, c_int, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


class QStateError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = lib().qstate_strerror(status).decode()
        super().__init__(f"{call} failed with status {status}: {msg}")
        self.status = status


def check(call: str, status: int) -> None:
    if status != QSTATE_OK:
        raise QStateError(call, status)
