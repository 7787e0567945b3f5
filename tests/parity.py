"""GPU-versus-reference parity harness (used by the gpu tests and the smoke check).

Both sides start from the same seeded inputs (workloads.py) and run the
whole workload independently: FP32 warm-up steps, the FP32 import, then the
quantized decode steps.  The CPU reference runs per head, so any subset of
the heads of a full-size batch can be checked one by one.

Contract per checked step and head:
  * codes bit-equal, except elements whose pre-rounding value lies within
    1e-6 (in code units) of a rounding threshold; those are counted, must be
    below 1e-5 of all checked elements, and the GPU head is then re-synced
    from the reference state (reference -> GPU only);
  * scales bit-equal;
  * o and the dequantized state within |a - b| <= 1e-5 + 1e-4 |b|;
  * the FP32 warm-up state bit-equal (the unquantized run is the FP32
    recurrence).
"""

from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import workloads as W
from exemption import check_rate, classify
from bit_recurrent_state_amd import qstate as Q

ATOL, RTOL = 1e-5, 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_rule(w: W.Workload):
    """(mode, threshold-or-fraction) of the decay-based allocation for w."""
    if w.bits_policy == "alpha_gt_0.99":
        return 0, 0.99
    if w.bits_policy == "rank_half":
        return 1, 0.5
    return None


def head_bits(w: W.Workload, seed=0, layer=0):
    """Per-head bits from the library and from the reference, which must agree."""
    rule = bits_rule(w)
    if rule is None:
        return np.full(w.H, 8, np.uint8)
    ret = W.head_retention(w, seed, layer)
    lib_bits = Q.qstate_bits_by_decay(ret, rule[0], rule[1])
    ref_bits = oracle.bits_by_decay(ret, rule[0], rule[1])
    assert np.array_equal(lib_bits, ref_bits), (lib_bits, ref_bits)
    return lib_bits


def block_bits(w: W.Workload, seed=0, layer=0):
    """Widths per head and 16-column block [H][dk/16].  "channel_half": per head
    the slower half of the G-channel groups INT8 (same rank rule, applied to
    the groups' mean channel retention), else the per-head widths."""
    nb = w.dk // 16
    if w.bits_policy != "channel_half":
        return np.repeat(head_bits(w, seed, layer)[:, None], nb, axis=1)
    ret = W.group_retention(w, seed, layer)
    out = np.empty((w.H, nb), np.uint8)
    for h in range(w.H):
        lib_bits = Q.qstate_bits_by_decay(ret[h], 1, 0.5)
        assert np.array_equal(lib_bits, oracle.bits_by_decay(ret[h], 1, 0.5))
        out[h] = np.repeat(lib_bits, w.G // 16)  # groups of G channels, G/16 blocks each
    return out


@dataclass
class Report:
    steps: int = 0
    elements: int = 0
    exempt: int = 0
    resyncs: int = 0
    max_o_err: float = 0.0
    max_s_err: float = 0.0
    first_exempt_step: int = -1
    notes: list = field(default_factory=list)


def _to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def _close(a, b):
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    err = np.abs(a64 - b64)
    return bool(np.all(err <= ATOL + RTOL * np.abs(b64))), float(err.max() if err.size else 0.0)


def _inputs_dev(inp):
    return [None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in inp]


class Run:
    """One workload instance on both sides."""

    def __init__(self, w: W.Workload, rounding=None, seed=0, layer=0, heads=None,
                 fp32_only=False, head_bits_override=None):
        self.w = w
        self.rounding = w.rounding if rounding is None else rounding
        self.seed, self.layer = seed, layer
        nb = w.dk // 16
        if head_bits_override is not None:
            hb = np.asarray(head_bits_override, np.uint8)
            self.bb = hb if hb.ndim == 2 else np.repeat(hb[:, None], nb, axis=1)
        else:
            self.bb = block_bits(w, seed, layer)
        self.hb = self.bb.max(axis=1)  # widest block per head (reporting only)
        uniform = bool(np.all(self.bb == self.bb[:, :1]))
        self.cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, self.rounding, False,
                            [int(x) for x in self.bb[:, 0]] if uniform else None, seed, layer,
                            w.axis, None if uniform else self.bb.tolist(), w.window,
                            w.window_merge, w.lrb_threshold)
        self.ocfg = oracle.cfg(w.B, w.H, w.dk, w.dv, w.G, w.mixer, self.rounding, seed, layer,
                               w.axis, w.window, w.window_merge, w.lrb_threshold)
        all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        self.heads = all_heads if heads is None else list(heads)
        self.rep = Report()
        self.t_in = 0  # next input step index
        self.fp32_only = fp32_only

    # ---- helpers -----------------------------------------------------------------
    def inputs(self, t):
        return W.step_inputs(self.w, t, self.seed, self.layer)

    def head_codes_slice(self, b, h):
        off = oracle.head_offset(self.ocfg, b, h, self.bb)
        n = oracle.head_code_bytes(self.ocfg, self.bb[h])
        return off, n

    # ---- pure-write window: the library's area (two key-side copies) -------------
    def _win_lib(self, codes_np, b, h, counter):
        """(a codes, b codes, scales) of head (b, h) in the library's window area as
        the step at `counter` reads it."""
        w = self.w
        W = w.window
        base = (oracle.codes_bytes(self.ocfg, self.bb) + 15) // 16 * 16
        whb = (w.dv * W + 2 * (W * w.dk + 8 * W) + 15) // 16 * 16
        area = codes_np[base + (b * w.H + h) * whb: base + (b * w.H + h + 1) * whb]
        cp = w.dv * W + (counter & 1) * (W * w.dk + 8 * W)
        return (area[:w.dv * W], area[cp:cp + W * w.dk],
                area[cp + W * w.dk:cp + W * w.dk + 8 * W])

    def _win_ref(self, win):
        w = self.w
        W = w.window
        return (win[:w.dv * W], win[w.dv * W:w.dv * W + W * w.dk],
                win[w.dv * W + W * w.dk:w.dv * W + W * w.dk + 8 * W])

    def _alpha_head(self, alpha, b, h):
        return alpha[b, h] if self.w.mixer in (W.GLA, W.KDA) else np.float32([alpha[b, h]])

    def _beta_head(self, beta, b, h):
        return 0.0 if beta is None else float(beta[b, h])

    # ---- phases ------------------------------------------------------------------
    def warmup_and_import(self):
        w = self.w
        zeros = torch.zeros(w.B * w.H * w.dv * w.dk, dtype=torch.float32, device="cuda")
        fcfg = Q.Config(w.B, w.H, w.dk, w.dv, 16, w.mixer, 0, True, None, self.seed, self.layer)
        f = Q.QState(fcfg)
        f.load_fp32(zeros)
        S_ref = {bh: np.zeros((w.dv, w.dk), np.float32) for bh in self.heads}
        for t in range(w.warmup):
            q, k, v, alpha, beta = self.inputs(t)
            dq, dk_, dv_, da, db = _inputs_dev((q, k, v, alpha, beta))
            f.step(dq, dk_, dv_, da, db, None)
            for (b, h) in self.heads:
                oracle.head_step_fp32(self.ocfg, S_ref[(b, h)], q[b, h], k[b, h], v[b, h],
                                      self._alpha_head(alpha, b, h), self._beta_head(beta, b, h))
        self.t_in = w.warmup
        S_gpu = torch.empty_like(zeros)
        f.store_fp32(S_gpu)
        torch.cuda.synchronize()
        Sg = _to_np(S_gpu).reshape(w.B, w.H, w.dv, w.dk)
        for (b, h) in self.heads:
            if not np.array_equal(Sg[b, h].view(np.uint32), S_ref[(b, h)].view(np.uint32)):
                bad = np.argwhere(Sg[b, h] != S_ref[(b, h)])
                raise AssertionError(f"FP32 warm-up state differs at head {(b, h)}, "
                                     f"{len(bad)} elements, first {bad[:3].tolist()}")
        f.close()
        self.S_fp32_ref = S_ref
        if self.fp32_only:
            return
        self.gpu = Q.QState(self.cfg)
        self.gpu.load_fp32(S_gpu)  # counter 0 -> 1
        self.ref, tdists, self.win = {}, {}, {}
        for (b, h) in self.heads:
            codes, scales, td = oracle.head_quantize(self.ocfg, b, h, self.bb[h],
                                                     S_ref[(b, h)], 0, want_tdist=True)
            self.ref[(b, h)] = (codes, scales)
            tdists[(b, h)] = td
            if w.window:
                self.win[(b, h)] = np.zeros(oracle.window_bytes(self.ocfg), np.uint8)
        torch.cuda.synchronize()
        self.compare(step=0, o_gpu=None, o_ref=None, tdists=tdists)

    def step(self, check=True):
        w = self.w
        q, k, v, alpha, beta = self.inputs(self.t_in)
        self.t_in += 1
        counter = self.gpu.step_counter
        dq, dk_, dv_, da, db = _inputs_dev((q, k, v, alpha, beta))
        o_dev = torch.full((w.B * w.H * w.dv,), float("nan"), dtype=torch.float32, device="cuda")
        self.gpu.step(dq, dk_, dv_, da, db, o_dev)
        o_ref, tdists = {}, {}
        for (b, h) in self.heads:
            codes, scales = self.ref[(b, h)]
            if w.window:
                o, _, td = oracle.head_step_pw(self.ocfg, b, h, self.bb[h], codes, scales,
                                               self.win[(b, h)], q[b, h], k[b, h], v[b, h],
                                               self._alpha_head(alpha, b, h),
                                               self._beta_head(beta, b, h), counter,
                                               want_tdist=True)
            else:
                o, _, td = oracle.head_step(self.ocfg, b, h, self.bb[h], codes, scales,
                                            q[b, h], k[b, h], v[b, h],
                                            self._alpha_head(alpha, b, h),
                                            self._beta_head(beta, b, h), counter,
                                            want_tdist=True)
            o_ref[(b, h)] = o
            tdists[(b, h)] = td
        torch.cuda.synchronize()
        if check:
            self.compare(step=counter, o_gpu=_to_np(o_dev).reshape(w.B, w.H, w.dv), o_ref=o_ref,
                         tdists=tdists)
        self.rep.steps += 1

    def compare(self, step, o_gpu, o_ref, tdists=None):
        w = self.w
        codes_g = _to_np(self.gpu.codes)
        scales_g = _to_np(self.gpu.scales).reshape(w.B, w.H, -1)
        for (b, h) in self.heads:
            bits = self.bb[h]
            off, n = self.head_codes_slice(b, h)
            cg = codes_g[off:off + n]
            cr, sr = self.ref[(b, h)]
            self.rep.elements += w.dv * w.dk
            if not np.array_equal(scales_g[b, h].ravel().view(np.uint32), sr.view(np.uint32)):
                bad = np.argwhere(scales_g[b, h].ravel() != sr)
                raise AssertionError(f"step {step} head {(b, h)}: {len(bad)} scales differ, "
                                     f"first {bad[:4].ravel().tolist()}")
            if not np.array_equal(cg, cr):
                self._exempt_or_fail(step, b, h, bits, cg, cr, tdists)
            if w.window:  # the window is part of the stored state: bit-exact
                counter = self.gpu.step_counter
                for name, g, r in zip(("a codes", "b codes", "scales"),
                                      self._win_lib(codes_g, b, h, counter),
                                      self._win_ref(self.win[(b, h)])):
                    if not np.array_equal(g, r):
                        bad = np.nonzero(g != r)[0]
                        raise AssertionError(f"step {step} head {(b, h)}: window {name} differ "
                                             f"at {len(bad)} bytes, first {bad[:4].tolist()}")
            if o_gpu is not None:
                ok, err = _close(o_gpu[b, h], o_ref[(b, h)])
                self.rep.max_o_err = max(self.rep.max_o_err, err)
                if not ok:
                    raise AssertionError(f"step {step} head {(b, h)}: o differs, max err {err}")
        check_rate(self.rep.exempt, self.rep.elements, f"step {step}")

    def _exempt_or_fail(self, step, b, h, bits, cg, cr, tdists):
        w = self.w
        a = _decode(cg, bits, w.dv, w.dk)
        r = _decode(cr, bits, w.dv, w.dk)
        bad = classify(a, r, tdists[(b, h)], f"step {step} head {(b, h)}")
        self.rep.exempt += len(bad)
        if self.rep.first_exempt_step < 0:
            self.rep.first_exempt_step = step
        # re-sync the GPU head from the reference (reference -> GPU only)
        off, n = self.head_codes_slice(b, h)
        self.gpu.codes[off:off + n] = torch.from_numpy(cr).cuda()
        self.rep.resyncs += 1

    def dequant_check(self):
        """Export (dequantized state) and readout against the reference."""
        w = self.w
        S = torch.empty(w.B * w.H * w.dv * w.dk, dtype=torch.float32, device="cuda")
        self.gpu.store_fp32(S)
        q, *_ = self.inputs(self.t_in)
        o = torch.empty(w.B * w.H * w.dv, dtype=torch.float32, device="cuda")
        self.gpu.readout(torch.from_numpy(q).cuda(), o)
        torch.cuda.synchronize()
        Sg = _to_np(S).reshape(w.B, w.H, w.dv, w.dk)
        og = _to_np(o).reshape(w.B, w.H, w.dv)
        counter = self.gpu.step_counter
        for (b, h) in self.heads:
            codes, scales = self.ref[(b, h)]
            if w.window:  # the full state: low-bit part plus the window's pairs
                Sr = oracle.head_window_state(self.ocfg, self.bb[h], codes, scales,
                                              self.win[(b, h)], counter)
                orr = oracle.head_window_readout(self.ocfg, self.bb[h], codes, scales,
                                                 self.win[(b, h)], counter, q[b, h])
            else:
                Sr = oracle.head_dequantize(self.ocfg, self.bb[h], codes, scales)
                orr = oracle.head_readout(self.ocfg, self.bb[h], codes, scales, q[b, h])
            assert np.array_equal(Sg[b, h], Sr), f"export differs at head {(b, h)}"
            ok, err = _close(og[b, h], orr)
            assert ok, f"readout differs at head {(b, h)}: {err}"
            self.rep.max_s_err = max(self.rep.max_s_err, float(np.abs(Sg[b, h] - Sr).max()))

    def close(self):
        if hasattr(self, "gpu"):
            self.gpu.close()


def _decode(codes: np.ndarray, bb: np.ndarray, dv: int, dk: int) -> np.ndarray:
    """Codes of one head in element order (i*dk + j), from per-block widths."""
    bb = np.asarray(bb).reshape(-1)
    row_bytes = int(np.sum(2 * bb.astype(np.int64)))
    rows = codes.reshape(dv, row_bytes)
    out = np.empty((dv, dk), np.int32)
    off = 0
    for q, bits in enumerate(bb):
        if bits == 8:
            out[:, 16 * q:16 * q + 16] = rows[:, off:off + 16].view(np.int8)
            off += 16
        else:
            blk = rows[:, off:off + 8]
            x = np.empty((dv, 16), np.int32)
            x[:, 0::2], x[:, 1::2] = blk & 0xF, blk >> 4
            x[x >= 8] -= 16
            out[:, 16 * q:16 * q + 16] = x
            off += 8
    return out.reshape(-1)
