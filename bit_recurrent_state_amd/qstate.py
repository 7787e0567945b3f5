"""Python binding of the qstate C ABI (include/qstate.h), same names.

Argument marshalling only: torch supplies device memory and the HIP stream,
every step of the path runs in the library's kernels.  Shapes and dtypes are
checked here so that a wrong tensor fails before it reaches the C ABI."""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import (BDR, GDN, GLA, KDA, KEY_AXIS, RTN, SCALAR, SR, VALUE_AXIS, QStateConfig, check,
                   lib)

__all__ = [
    "GDN", "GLA", "SCALAR", "KDA", "RTN", "SR", "BDR", "VALUE_AXIS", "KEY_AXIS", "Config",
    "QState",
    "qstate_state_bytes", "qstate_create", "qstate_load_fp32", "qstate_step",
    "qstate_readout", "qstate_store_fp32", "qstate_get_step", "qstate_set_step",
    "qstate_destroy", "qstate_bits_by_decay",
]


@dataclass
class Config:
    batch: int
    heads: int
    dk: int
    dv: int
    group: int = 64
    mixer: int = GDN
    rounding: int = RTN
    fp32_state: bool = False
    head_bits: Optional[Sequence[int]] = None
    seed: int = 0
    layer: int = 0
    group_axis: int = VALUE_AXIS
    channel_bits: Optional[Sequence[Sequence[int]]] = None  # [heads][dk/16], overrides head_bits
    window: int = 0  # pure-write window length W (0, 4, 8 or 16)
    window_merge: int = 0  # 0 pure-write window, 1 low-rank bypass (merge every W steps)
    lrb_threshold: float = 0.5  # low-rank bypass: merge |m| >= threshold * group scale

    def to_c(self):
        """(QStateConfig, keep-alive buffers)."""
        keep = []
        ptr = cptr = None
        if self.head_bits is not None:
            hb = (ctypes.c_uint8 * self.heads)(*[int(x) for x in self.head_bits])
            ptr = ctypes.cast(hb, ctypes.POINTER(ctypes.c_uint8))
            keep.append(hb)
        if self.channel_bits is not None:
            flat = np.asarray(self.channel_bits, np.uint8).reshape(-1)
            if flat.size != self.heads * (self.dk // 16):
                raise ValueError("channel_bits: expected [heads][dk/16] widths")
            cb = (ctypes.c_uint8 * flat.size)(*[int(x) for x in flat])
            cptr = ctypes.cast(cb, ctypes.POINTER(ctypes.c_uint8))
            keep.append(cb)
        c = QStateConfig(self.batch, self.heads, self.dk, self.dv, self.group, self.mixer,
                         self.rounding, int(bool(self.fp32_state)), ptr, self.seed, self.layer,
                         self.group_axis, cptr, self.window, self.window_merge,
                         self.lrb_threshold)
        return c, keep

    def bits(self) -> np.ndarray:
        """Widths per head and 16-column block, [heads][dk/16] (32 for an FP32 state)."""
        nb = self.dk // 16
        if self.fp32_state:
            return np.full((self.heads, nb), 32, np.int64)
        if self.channel_bits is not None:
            return np.asarray(self.channel_bits, np.int64).reshape(self.heads, nb)
        if self.head_bits is None:
            return np.full((self.heads, nb), 8, np.int64)
        return np.repeat(np.asarray(self.head_bits, np.int64)[:, None], nb, axis=1)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype, numel: int):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name}: expected contiguous {dtype} with {numel} elements, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    return ctypes.c_void_p(t.data_ptr())


def qstate_state_bytes(cfg: Config):
    c, _keep = cfg.to_c()
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    check("qstate_state_bytes", lib().qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb),
                                                          ctypes.byref(sb)))
    return cb.value, sb.value


def qstate_create(cfg: Config, codes: torch.Tensor, scales: Optional[torch.Tensor]):
    cb, sb = qstate_state_bytes(cfg)
    if cfg.fp32_state:
        pc = _dev(codes, "state", torch.float32, cb // 4)
        ps = None
    else:
        pc = _dev(codes, "codes", torch.uint8, cb)
        ps = _dev(scales, "scales", torch.float32, sb // 4)
    c, _keep = cfg.to_c()
    h = ctypes.c_void_p()
    check("qstate_create", lib().qstate_create(ctypes.byref(c), pc, ps, ctypes.byref(h)))
    return h


def qstate_load_fp32(h, S: torch.Tensor, cfg: Config, stream=None):
    n = cfg.batch * cfg.heads * cfg.dv * cfg.dk
    check("qstate_load_fp32", lib().qstate_load_fp32(h, _dev(S, "S", torch.float32, n),
                                                      _stream(stream)))


def qstate_step(h, cfg: Config, q, k, v, alpha, beta=None, o=None, stream=None):
    bh = cfg.batch * cfg.heads
    na = bh * cfg.dk if cfg.mixer in (GLA, KDA) else bh
    args = (
        _dev(q, "q", torch.float32, bh * cfg.dk), _dev(k, "k", torch.float32, bh * cfg.dk),
        _dev(v, "v", torch.float32, bh * cfg.dv), _dev(alpha, "alpha", torch.float32, na),
        None if cfg.mixer == GLA else _dev(beta, "beta", torch.float32, bh),
        _dev(o, "o", torch.float32, bh * cfg.dv),
    )
    check("qstate_step", lib().qstate_step(h, *args, _stream(stream)))


def qstate_readout(h, cfg: Config, q, o, stream=None):
    bh = cfg.batch * cfg.heads
    check("qstate_readout", lib().qstate_readout(h, _dev(q, "q", torch.float32, bh * cfg.dk),
                                                  _dev(o, "o", torch.float32, bh * cfg.dv),
                                                  _stream(stream)))


def qstate_store_fp32(h, cfg: Config, S, stream=None):
    n = cfg.batch * cfg.heads * cfg.dv * cfg.dk
    check("qstate_store_fp32", lib().qstate_store_fp32(h, _dev(S, "S", torch.float32, n),
                                                        _stream(stream)))


def qstate_get_step(h) -> int:
    s = ctypes.c_uint64()
    check("qstate_get_step", lib().qstate_get_step(h, ctypes.byref(s)))
    return s.value


def qstate_set_step(h, step: int) -> None:
    check("qstate_set_step", lib().qstate_set_step(h, step))


def qstate_destroy(h) -> None:
    check("qstate_destroy", lib().qstate_destroy(h))


def qstate_bits_by_decay(retention, mode: int, thr_or_frac: float, lo_bits: int = 4,
                         hi_bits: int = 8) -> np.ndarray:
    r = np.ascontiguousarray(retention, dtype=np.float32)
    out = np.zeros(r.size, np.uint8)
    check("qstate_bits_by_decay",
          lib().qstate_bits_by_decay(r.ctypes.data_as(ctypes.c_void_p), r.size, mode,
                                     thr_or_frac, lo_bits, hi_bits,
                                     out.ctypes.data_as(ctypes.c_void_p)))
    return out


class QState:
    """A handle plus the torch device buffers it works on (caller-owned memory)."""

    def __init__(self, cfg: Config, device="cuda"):
        self.cfg = cfg
        cb, sb = qstate_state_bytes(cfg)
        if cfg.fp32_state:
            self.codes = torch.zeros(cb // 4, dtype=torch.float32, device=device)
            self.scales = None
        else:
            self.codes = torch.zeros(cb, dtype=torch.uint8, device=device)
            self.scales = torch.zeros(sb // 4, dtype=torch.float32, device=device)
        self.handle = qstate_create(cfg, self.codes, self.scales)

    def load_fp32(self, S, stream=None):
        qstate_load_fp32(self.handle, S, self.cfg, stream)

    def step(self, q, k, v, alpha, beta=None, o=None, stream=None):
        qstate_step(self.handle, self.cfg, q, k, v, alpha, beta, o, stream)

    def readout(self, q, o, stream=None):
        qstate_readout(self.handle, self.cfg, q, o, stream)

    def store_fp32(self, S, stream=None):
        qstate_store_fp32(self.handle, self.cfg, S, stream)

    @property
    def step_counter(self) -> int:
        return qstate_get_step(self.handle)

    @step_counter.setter
    def step_counter(self, value: int) -> None:
        qstate_set_step(self.handle, value)

    def close(self):
        if self.handle is not None:
            qstate_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
