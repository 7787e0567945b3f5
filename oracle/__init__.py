"""CPU reference of the quantized recurrent-state decode step (numpy wrapper).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The product package never imports it.

The arithmetic lives in ``oracle.cpp`` (plain single-threaded C++); this
module marshals numpy arrays to it and builds the shared object on demand.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")
# A separately built copy (e.g. the sanitizer build of tests/test_sanitizers.py)
# may be loaded instead by naming it in QSTATE_ORACLE_LIB.
LIB_OVERRIDE = os.environ.get("QSTATE_ORACLE_LIB")

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2
VALUE_AXIS, KEY_AXIS = 0, 1


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (no fast-math, no FP contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
        os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "oracle.h"))
    ):
        tmp = LIB + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-o", tmp, SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


class Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("G", ctypes.c_int32), ("mixer", ctypes.c_int32),
                ("rounding", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("layer", ctypes.c_uint32), ("axis", ctypes.c_int32),
                ("window", ctypes.c_int32), ("window_merge", ctypes.c_int32),
                ("lrb_threshold", ctypes.c_float)]


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(LIB_OVERRIDE if LIB_OVERRIDE else build())
        u64, u32, i32, f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float
        cp = ctypes.POINTER(Cfg)
        sig = {
            "oracle_splitmix64_output": (u64, [u64]),
            "oracle_fmix32": (u32, [u32]),
            "oracle_lcg16x2": (u32, [u32]),
            "oracle_head_key": (u32, [u64, u32, u64, u32, u32]),
            "oracle_sr_bits": (u32, [u32, u64]),
            "oracle_dot": (f32, [_P, _P, i32]),
            "oracle_group_scale": (None, [f32, i32, _P, _P]),
            "oracle_round_rtn": (i32, [f32, f32]),
            "oracle_round_sr": (i32, [f32, f32, u32, i32]),
            "oracle_round_bdr": (i32, [f32, f32, f32, f32, i32]),
            "oracle_threshold_distance": (ctypes.c_double, [f32, f32, i32, u32, i32]),
            "oracle_codes_bytes": (ctypes.c_size_t, [cp, _P]),
            "oracle_head_offset": (ctypes.c_size_t, [cp, _P, i32, i32]),
            "oracle_get_code": (i32, [_P, i32, ctypes.c_int64]),
            "oracle_set_code": (None, [_P, i32, ctypes.c_int64, i32]),
            "oracle_head_step": (None, [cp, i32, i32, _P, _P, _P, _P, _P, _P, _P, f32,
                                        _P, u64, _P, _P]),
            "oracle_head_step_fp32": (None, [cp, _P, _P, _P, _P, _P, f32, _P]),
            "oracle_head_quantize": (None, [cp, i32, i32, _P, _P, _P, _P, u64, _P]),
            "oracle_head_dequantize": (None, [cp, _P, _P, _P, _P]),
            "oracle_head_readout": (None, [cp, _P, _P, _P, _P, _P]),
            "oracle_step": (None, [cp, _P, _P, _P, _P, _P, _P, _P, _P, _P, u64]),
            "oracle_step_fp32": (None, [cp, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_step_heads": (None, [cp, _P, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, u64]),
            "oracle_step_fp32_heads": (None, [cp, i32, _P, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_quantize_heads": (None, [cp, _P, i32, _P, _P, _P, _P, u64]),
            "oracle_quantize": (None, [cp, _P, _P, _P, _P, u64]),
            "oracle_dequantize": (None, [cp, _P, _P, _P, _P]),
            "oracle_readout": (None, [cp, _P, _P, _P, _P, _P]),
            "oracle_bits_by_decay": (i32, [_P, i32, i32, f32, ctypes.c_uint8,
                                           ctypes.c_uint8, _P]),
            "oracle_fp8_decode": (f32, [ctypes.c_uint8]),
            "oracle_fp8_encode": (ctypes.c_uint8, [f32]),
            "oracle_window_bytes": (ctypes.c_size_t, [cp]),
            "oracle_head_step_pw": (None, [cp, i32, i32, _P, _P, _P, _P, _P, _P, _P, _P, f32,
                                           _P, u64, _P, _P]),
            "oracle_head_window_state": (None, [cp, _P, _P, _P, _P, u64, _P]),
            "oracle_head_window_readout": (None, [cp, _P, _P, _P, _P, u64, _P, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def cfg(B, H, dk, dv, G, mixer=GDN, rounding=RTN, seed=0, layer=0, axis=VALUE_AXIS,
        window=0, window_merge=0, lrb_threshold=0.5) -> Cfg:
    return Cfg(B, H, dk, dv, G, mixer, rounding, seed, layer, axis, window, window_merge,
               lrb_threshold)


def scales_shape(c: Cfg):
    """Per-head scale array: [dv][dk/G] (value-axis groups) or [dv/G][dk] (key-axis)."""
    return (c.dv // c.G, c.dk) if c.axis == KEY_AXIS else (c.dv, c.dk // c.G)


def head_bits_array(c: Cfg, head_bits=None) -> np.ndarray:
    """Bit widths per head and 16-column block, [H][dk/16]: from None (all
    INT8), one width per head [H], or per block [H][dk/16]."""
    nb = c.dk // 16
    if head_bits is None:
        return np.full((c.H, nb), 8, dtype=np.uint8)
    hb = np.asarray(head_bits, dtype=np.uint8)
    if hb.ndim == 1:
        assert hb.shape == (c.H,)
        hb = np.repeat(hb[:, None], nb, axis=1)
    assert hb.shape == (c.H, nb)
    return np.ascontiguousarray(hb)


def block_bits(c: Cfg, bits) -> np.ndarray:
    """Widths of one head's 16-column blocks, from one width or a block list."""
    nb = c.dk // 16
    bb = np.asarray(bits, dtype=np.uint8).reshape(-1)
    if bb.size == 1:
        bb = np.full(nb, bb[0], np.uint8)
    assert bb.shape == (nb,)
    return np.ascontiguousarray(bb)


def head_code_bytes(c: Cfg, bits) -> int:
    """Code bytes of one head with the given width(s)."""
    return int(c.dv * np.sum(block_bits(c, bits).astype(np.int64) * 2))


# ---- scalar pieces -------------------------------------------------------

def splitmix64_output(z: int) -> int:
    return lib().oracle_splitmix64_output(z)


def fmix32(h: int) -> int:
    return lib().oracle_fmix32(h)


def lcg16x2(w: int) -> int:
    return lib().oracle_lcg16x2(w)


def head_key(seed, layer, step, b, h) -> int:
    return lib().oracle_head_key(seed, layer, step, b, h)


def sr_bits(key: int, element: int) -> int:
    return lib().oracle_sr_bits(key, element)


def dot(x, y) -> float:
    x, y = _f32(x), _f32(y)
    assert x.shape == y.shape and x.ndim == 1
    return lib().oracle_dot(_ptr(x), _ptr(y), x.size)


def group_scale(m: float, r: int):
    s = np.zeros(1, np.float32)
    inv = np.zeros(1, np.float32)
    lib().oracle_group_scale(m, r, _ptr(s), _ptr(inv))
    return s[0], inv[0]


def round_rtn(x: float, inv: float) -> int:
    return lib().oracle_round_rtn(x, inv)


def round_sr(x: float, inv: float, r16: int, bits: int) -> int:
    return lib().oracle_round_sr(x, inv, r16, bits)


def round_bdr(x: float, inv: float, s_new: float, prev: float, r: int) -> int:
    return lib().oracle_round_bdr(x, inv, s_new, prev, r)


def threshold_distance(x: float, inv: float, stochastic: bool, r16: int, bits: int) -> float:
    """Distance in code units from x*inv to the nearest point where the code changes."""
    return lib().oracle_threshold_distance(x, inv, int(bool(stochastic)), r16, bits)


def codes_bytes(c: Cfg, head_bits=None) -> int:
    hb = head_bits_array(c, head_bits)
    return lib().oracle_codes_bytes(ctypes.byref(c), _ptr(hb))


def head_offset(c: Cfg, b: int, h: int, head_bits=None) -> int:
    hb = head_bits_array(c, head_bits)
    return lib().oracle_head_offset(ctypes.byref(c), _ptr(hb), b, h)


def get_code(head_codes: np.ndarray, bits: int, e: int) -> int:
    return lib().oracle_get_code(_ptr(head_codes), bits, e)


def unpack_head(c: Cfg, head_codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes of one head as int [dv, dk] (element-by-element, slow)."""
    n = c.dv * c.dk
    out = np.empty(n, np.int32)
    L = lib()
    p = _ptr(head_codes)
    for e in range(n):
        out[e] = L.oracle_get_code(p, bits, e)
    return out.reshape(c.dv, c.dk)


# ---- one head --------------------------------------------------------------

def head_step(c: Cfg, b, h, bits, codes, scales, q, k, v, alpha, beta, step,
              want_pre=False, want_tdist=False):
    """One quantized step of one head; codes/scales (numpy) are updated in place.

    Returns (o, pre, tdist) with pre/tdist None unless requested."""
    assert codes.dtype == np.uint8 and codes.flags.c_contiguous
    assert scales.dtype == np.float32 and scales.flags.c_contiguous
    bb = block_bits(c, bits)
    assert codes.size == head_code_bytes(c, bb)
    assert scales.size == int(np.prod(scales_shape(c)))
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    assert q.size == c.dk and k.size == c.dk and v.size == c.dv
    assert alpha.size == (c.dk if c.mixer in (GLA, KDA) else 1)
    o = np.zeros(c.dv, np.float32)
    pre = np.zeros((c.dv, c.dk), np.float32) if want_pre else None
    tdist = np.zeros((c.dv, c.dk), np.float64) if want_tdist else None
    lib().oracle_head_step(ctypes.byref(c), b, h, _ptr(bb), _ptr(codes), _ptr(scales), _ptr(q),
                           _ptr(k), _ptr(v), _ptr(alpha), float(beta), _ptr(o), step,
                           _ptr(pre), _ptr(tdist))
    return o, pre, tdist


def head_step_fp32(c: Cfg, S, q, k, v, alpha, beta):
    assert S.dtype == np.float32 and S.flags.c_contiguous and S.size == c.dv * c.dk
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    o = np.zeros(c.dv, np.float32)
    lib().oracle_head_step_fp32(ctypes.byref(c), _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(alpha), float(beta), _ptr(o))
    return o


def head_quantize(c: Cfg, b, h, bits, S, step, want_tdist=False):
    S = _f32(S)
    assert S.size == c.dv * c.dk
    bb = block_bits(c, bits)
    codes = np.zeros(head_code_bytes(c, bb), np.uint8)
    scales = np.zeros(int(np.prod(scales_shape(c))), np.float32)
    tdist = np.zeros((c.dv, c.dk), np.float64) if want_tdist else None
    lib().oracle_head_quantize(ctypes.byref(c), b, h, _ptr(bb), _ptr(S), _ptr(codes),
                               _ptr(scales), step, _ptr(tdist))
    return codes, scales, tdist


def head_dequantize(c: Cfg, bits, codes, scales):
    S = np.zeros((c.dv, c.dk), np.float32)
    lib().oracle_head_dequantize(ctypes.byref(c), _ptr(block_bits(c, bits)),
                                 _ptr(np.ascontiguousarray(codes)),
                                 _ptr(_f32(scales)), _ptr(S))
    return S


def head_readout(c: Cfg, bits, codes, scales, q):
    o = np.zeros(c.dv, np.float32)
    lib().oracle_head_readout(ctypes.byref(c), _ptr(block_bits(c, bits)),
                              _ptr(np.ascontiguousarray(codes)),
                              _ptr(_f32(scales)), _ptr(_f32(q)), _ptr(o))
    return o


# ---- whole batch -------------------------------------------------------------

def step(c: Cfg, head_bits, codes, scales, q, k, v, alpha, beta, t):
    """Quantized step over all heads, in place on codes/scales; returns o."""
    hb = head_bits_array(c, head_bits)
    assert codes.dtype == np.uint8 and codes.size == codes_bytes(c, hb)
    assert scales.dtype == np.float32 and scales.flags.c_contiguous
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    beta = None if beta is None else _f32(beta)
    o = np.zeros((c.B, c.H, c.dv), np.float32)
    lib().oracle_step(ctypes.byref(c), _ptr(hb), _ptr(codes), _ptr(scales), _ptr(q), _ptr(k),
                      _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), t)
    return o


def step_fp32(c: Cfg, S, q, k, v, alpha, beta):
    assert S.dtype == np.float32 and S.flags.c_contiguous
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    beta = None if beta is None else _f32(beta)
    o = np.zeros((c.B, c.H, c.dv), np.float32)
    lib().oracle_step_fp32(ctypes.byref(c), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                           _ptr(beta), _ptr(o))
    return o


def quantize(c: Cfg, head_bits, S, t):
    hb = head_bits_array(c, head_bits)
    S = _f32(S)
    codes = np.zeros(codes_bytes(c, hb), np.uint8)
    scales = np.zeros((c.B, c.H) + scales_shape(c), np.float32)
    lib().oracle_quantize(ctypes.byref(c), _ptr(hb), _ptr(S), _ptr(codes), _ptr(scales), t)
    return codes, scales


def dequantize(c: Cfg, head_bits, codes, scales):
    hb = head_bits_array(c, head_bits)
    S = np.zeros((c.B, c.H, c.dv, c.dk), np.float32)
    lib().oracle_dequantize(ctypes.byref(c), _ptr(hb), _ptr(codes), _ptr(_f32(scales)), _ptr(S))
    return S


def readout(c: Cfg, head_bits, codes, scales, q):
    hb = head_bits_array(c, head_bits)
    o = np.zeros((c.B, c.H, c.dv), np.float32)
    lib().oracle_readout(ctypes.byref(c), _ptr(hb), _ptr(codes), _ptr(_f32(scales)),
                         _ptr(_f32(q)), _ptr(o))
    return o


# ---- listed heads of a batch (thread-safe on disjoint lists) --------------------

def _heads(heads):
    return np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1))


def step_heads(c: Cfg, head_bits, heads, codes, scales, q, k, v, alpha, beta, t, o=None):
    """Quantized step of the listed heads (indices b*H + h) of full-batch arrays,
    in place on codes/scales; o [B][H][dv] receives their readouts."""
    hb = head_bits_array(c, head_bits)
    idx = _heads(heads)
    assert codes.dtype == np.uint8 and codes.flags.c_contiguous
    assert scales.dtype == np.float32 and scales.flags.c_contiguous
    for a in (q, k, v, alpha) + (() if beta is None else (beta,)):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    lib().oracle_step_heads(ctypes.byref(c), _ptr(hb), idx.size, _ptr(idx), _ptr(codes),
                            _ptr(scales), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(o), t)


def step_fp32_heads(c: Cfg, heads, S, q, k, v, alpha, beta, o=None):
    idx = _heads(heads)
    assert S.dtype == np.float32 and S.flags.c_contiguous
    lib().oracle_step_fp32_heads(ctypes.byref(c), idx.size, _ptr(idx), _ptr(S), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o))


def quantize_heads(c: Cfg, head_bits, heads, S, codes, scales, t):
    hb = head_bits_array(c, head_bits)
    idx = _heads(heads)
    assert S.dtype == np.float32 and S.flags.c_contiguous
    lib().oracle_quantize_heads(ctypes.byref(c), _ptr(hb), idx.size, _ptr(idx), _ptr(S),
                                _ptr(codes), _ptr(scales), t)


def bits_by_decay(retention, mode, thr_or_frac, lo=4, hi=8):
    ret = _f32(retention)
    out = np.zeros(ret.size, np.uint8)
    rc = lib().oracle_bits_by_decay(_ptr(ret), ret.size, mode, thr_or_frac, lo, hi, _ptr(out))
    if rc != 0:
        raise ValueError("bits_by_decay: bad arguments")
    return out


# ---- pure-write window ---------------------------------------------------------

def fp8_decode(code: int) -> float:
    return lib().oracle_fp8_decode(code)


def fp8_encode(x: float) -> int:
    return lib().oracle_fp8_encode(x)


def window_bytes(c: Cfg) -> int:
    return lib().oracle_window_bytes(ctypes.byref(c))


def head_step_pw(c: Cfg, b, h, bits, codes, scales, window, q, k, v, alpha, beta, step,
                 want_pre=False, want_tdist=False):
    """One quantized step of one head with its pure-write window (updated in place)."""
    bb = block_bits(c, bits)
    assert codes.size == head_code_bytes(c, bb) and window.size == window_bytes(c)
    assert window.dtype == np.uint8 and window.flags.c_contiguous
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    o = np.zeros(c.dv, np.float32)
    pre = np.zeros((c.dv, c.dk), np.float32) if want_pre else None
    tdist = np.zeros((c.dv, c.dk), np.float64) if want_tdist else None
    lib().oracle_head_step_pw(ctypes.byref(c), b, h, _ptr(bb), _ptr(codes), _ptr(scales),
                              _ptr(window), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), float(beta),
                              _ptr(o), step, _ptr(pre), _ptr(tdist))
    return o, pre, tdist


def head_window_state(c: Cfg, bits, codes, scales, window, step):
    S = np.zeros((c.dv, c.dk), np.float32)
    lib().oracle_head_window_state(ctypes.byref(c), _ptr(block_bits(c, bits)),
                                   _ptr(np.ascontiguousarray(codes)), _ptr(_f32(scales)),
                                   _ptr(np.ascontiguousarray(window)), step, _ptr(S))
    return S


def head_window_readout(c: Cfg, bits, codes, scales, window, step, q):
    o = np.zeros(c.dv, np.float32)
    lib().oracle_head_window_readout(ctypes.byref(c), _ptr(block_bits(c, bits)),
                                     _ptr(np.ascontiguousarray(codes)), _ptr(_f32(scales)),
                                     _ptr(np.ascontiguousarray(window)), step, _ptr(_f32(q)),
                                     _ptr(o))
    return o
