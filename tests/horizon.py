"""Long-horizon GPU-versus-reference parity at the workloads' own step counts.

Both sides start from the same seeded inputs (workloads.py) and run the
whole workload independently: FP32 warm-up, the import (counter 0), then T
quantized decode steps.  The library runs every head of the batch at its
real launch size; the CPU reference runs a set of tracked heads, stepped on
host threads (heads are independent and the reference is single-threaded
per head, so disjoint head lists may run at once).

Checked on every tracked head at every step (the parity contract):
  * codes bit-equal, except one-code differences within 1e-6 code units of a
    threshold (tests/exemption.py), counted against 1e-5 of the elements;
  * scales bit-equal;
  * o within |a - b| <= 1e-5 + 1e-4 |b|;
  * the FP32 warm-up state bit-equal before the import.
"Every head" sets are tracked through the import and step 1 and then
narrowed to the sampled heads.

The reference never reads GPU data.  An exempted difference overwrites that
head's GPU codes with the reference's (reference -> GPU), so the trajectories
stay comparable; the report gives the first such step, and with none the
two trajectories are bit-identical through step T ("free-running: bit-exact").
"""

from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import workloads as W
from bit_recurrent_state_amd import qstate as Q
from exemption import ParityError, check_rate, classify
from parity import ATOL, RTOL, _decode, block_bits, log


def host_threads() -> int:
    """Worker threads for the reference: the host cores we may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class HorizonReport:
    workload: str = ""
    rounding: int = 0
    layer: int = 0
    steps: int = 0
    heads_tracked: int = 0
    heads_every: int = 0
    head_steps: int = 0
    elements: int = 0
    exempt: int = 0
    first_exempt_step: int = -1
    max_o_err: float = 0.0
    seconds: float = 0.0
    notes: list = field(default_factory=list)

    @property
    def free_running(self) -> str:
        if self.first_exempt_step < 0:
            return f"bit-exact through step {self.steps}"
        return f"first divergence (near-threshold, re-synced) at step {self.first_exempt_step}"


class _Prefetch:
    """Inputs of upcoming steps drawn on host threads ahead of use."""

    def __init__(self, w, seed, layer, first, last, ahead=12, workers=8):
        self.w, self.seed, self.layer = w, seed, layer
        self.next, self.last, self.ahead = first, last, ahead
        self.ex = ThreadPoolExecutor(max_workers=workers)
        self.fut = {}
        self._fill()

    def _fill(self):
        while len(self.fut) < self.ahead and self.next < self.last:
            t = self.next
            self.fut[t] = self.ex.submit(W.step_inputs, self.w, t, self.seed, self.layer)
            self.next += 1

    def get(self, t):
        x = self.fut.pop(t).result()
        self._fill()
        return tuple(None if a is None else np.ascontiguousarray(a) for a in x)

    def close(self):
        self.ex.shutdown(wait=True, cancel_futures=True)


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


class Horizon:
    """One workload instance (one layer) on both sides, tracked heads compared every step."""

    def __init__(self, w: W.Workload, rounding=None, seed=0, layer=0, tracked=None, every=None,
                 threads=None):
        assert w.window == 0, "pair buffers are checked by tests/parity.py"
        self.w = w
        self.rounding = w.rounding if rounding is None else rounding
        self.seed, self.layer = seed, layer
        self.bb = block_bits(w, seed, layer)  # library and reference allocation agree
        uniform = bool(np.all(self.bb == self.bb[:, :1]))
        self.cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, self.rounding, False,
                            [int(x) for x in self.bb[:, 0]] if uniform else None, seed, layer,
                            w.axis, None if uniform else self.bb.tolist())
        self.ocfg = oracle.cfg(w.B, w.H, w.dk, w.dv, w.G, w.mixer, self.rounding, seed, layer,
                               w.axis)
        n = w.B * w.H
        self.tracked = np.arange(n) if tracked is None else np.unique(np.asarray(tracked))
        self.every = (np.arange(n) if every == "all" else
                      np.unique(np.concatenate([self.tracked, np.asarray(every or [], int)])))
        self.threads = threads or host_threads()
        self.pool = ThreadPoolExecutor(max_workers=self.threads)
        # layout: per-head code bytes and offsets, scales per head
        row_bytes = 2 * self.bb.astype(np.int64).sum(axis=1)  # bytes of a value row, per h
        hbytes = w.dv * row_bytes
        self.per_b = int(hbytes.sum())
        self.hoff = np.concatenate([[0], np.cumsum(hbytes)[:-1]])
        self.hbytes = hbytes
        self.n_scales = int(np.prod(oracle.scales_shape(self.ocfg)))
        for (b, h) in ((0, 0), (w.B - 1, w.H - 1)):
            assert self._off(b * w.H + h) == oracle.head_offset(self.ocfg, b, h, self.bb)
        self.rep = HorizonReport(w.name, self.rounding, layer)

    # ---- layout ---------------------------------------------------------------------
    def _off(self, bh):
        b, h = divmod(int(bh), self.w.H)
        return b * self.per_b + int(self.hoff[h])

    def _code_index(self, heads):
        return np.concatenate([np.arange(self._off(bh), self._off(bh) + self.hbytes[bh % self.w.H])
                               for bh in heads]) if len(heads) else np.zeros(0, np.int64)

    def _scale_index(self, heads):
        ns = self.n_scales
        return (np.asarray(heads, np.int64)[:, None] * ns + np.arange(ns)[None, :]).ravel()

    def _set(self, heads):
        """Gather indices (device and host) of a head set."""
        heads = np.asarray(heads, np.int64)
        ci, si = self._code_index(heads), self._scale_index(heads)
        oi = (heads[:, None] * self.w.dv + np.arange(self.w.dv)[None, :]).ravel()
        full = len(heads) == self.w.B * self.w.H
        return {"heads": heads, "full": full, "ci": ci, "si": si, "oi": oi,
                "ci_d": None if full else torch.from_numpy(ci).cuda(),
                "si_d": None if full else torch.from_numpy(si).cuda(),
                "oi_d": None if full else torch.from_numpy(oi).cuda()}

    def _gather(self, t: torch.Tensor, idx_d):
        return (t if idx_d is None else t.index_select(0, idx_d)).cpu().numpy()

    # ---- the reference on host threads ------------------------------------------------
    def _chunks(self, heads):
        k = min(self.threads, max(1, len(heads)))
        return [c for c in np.array_split(np.asarray(heads, np.int32), k) if c.size]

    def _par(self, fn, heads):
        list(self.pool.map(fn, self._chunks(heads)))

    # ---- phases ---------------------------------------------------------------------
    def run(self, steps: int):
        t0 = time.time()
        w = self.w
        pre = _Prefetch(w, self.seed, self.layer, 0, w.warmup + steps)
        try:
            self._warmup_and_import(pre)
            o_dev = torch.empty(w.B * w.H * w.dv, dtype=torch.float32, device="cuda")
            o_ref = np.zeros(w.B * w.H * w.dv, np.float32)
            for t in range(1, steps + 1):
                active = self.S_every if t == 1 else self.S_tracked
                self._step(pre.get(w.warmup + t - 1), t, active, o_dev, o_ref)
                if t in (1, steps) or t % 128 == 0:
                    log(f"  step {t}/{steps}: heads {len(active['heads'])} exempt "
                        f"{self.rep.exempt} max|o err| {self.rep.max_o_err:.3g} "
                        f"({time.time() - t0:.0f} s)")
            self._final_check(pre_q=W.step_inputs(w, w.warmup + steps, self.seed, self.layer)[0])
        finally:
            pre.close()
            self.pool.shutdown(wait=True)
            if hasattr(self, "gpu"):
                self.gpu.close()
        self.rep.steps = steps
        self.rep.seconds = time.time() - t0
        return self.rep

    def _warmup_and_import(self, pre):
        w = self.w
        n = w.B * w.H * w.dv * w.dk
        f = Q.QState(Q.Config(w.B, w.H, w.dk, w.dv, 16, w.mixer, 0, True, None, self.seed,
                              self.layer))
        f.load_fp32(torch.zeros(n, dtype=torch.float32, device="cuda"))
        S_ref = np.zeros(n, np.float32)  # only the heads of `every` are touched
        every = self.every
        for t in range(w.warmup):
            q, k, v, alpha, beta = pre.get(t)
            f.step(*map(_dev, (q, k, v, alpha, beta)))
            self._par(lambda hs: oracle.step_fp32_heads(self.ocfg, hs, S_ref, q, k, v, alpha,
                                                        beta), every)
        S_gpu = torch.empty(n, dtype=torch.float32, device="cuda")
        f.store_fp32(S_gpu)
        f.close()
        hs = w.dv * w.dk
        sidx = (every[:, None] * hs + np.arange(hs)[None, :]).ravel()
        full = len(every) == w.B * w.H
        Sg = (S_gpu if full else S_gpu.index_select(0, torch.from_numpy(sidx).cuda())).cpu().numpy()
        if not np.array_equal(Sg.view(np.uint32), S_ref[sidx].view(np.uint32)):
            bad = np.nonzero(Sg.view(np.uint32) != S_ref[sidx].view(np.uint32))[0]
            raise ParityError(f"FP32 warm-up state differs at {bad.size} elements, first head "
                              f"{every[bad[0] // hs]}")
        # import (counter 0) on both sides
        self.gpu = Q.QState(self.cfg)
        self.gpu.load_fp32(S_gpu)
        del S_gpu
        cb, sb = Q.qstate_state_bytes(self.cfg)
        self.codes = np.zeros(cb, np.uint8)
        self.scales = np.zeros(sb // 4, np.float32)
        self._par(lambda hs_: oracle.quantize_heads(self.ocfg, self.bb, hs_, S_ref, self.codes,
                                                    self.scales, 0), every)
        self.S_every = self._set(every)
        self.S_tracked = self._set(self.tracked)
        self.rep.heads_every = len(every)
        self.rep.heads_tracked = len(self.tracked)
        torch.cuda.synchronize()
        self._compare(0, self.S_every, None, None, ("import", S_ref))

    def _step(self, inputs, t, S, o_dev, o_ref):
        q, k, v, alpha, beta = inputs
        counter = self.gpu.step_counter
        assert counter == t
        self.gpu.step(*map(_dev, (q, k, v, alpha, beta)), o_dev)
        # pre-step copies of the active heads (to recompute threshold distances)
        pre_codes, pre_scales = self.codes[S["ci"]], self.scales[S["si"]]
        self._par(lambda hs: oracle.step_heads(self.ocfg, self.bb, hs, self.codes, self.scales,
                                               q, k, v, alpha, beta, t, o_ref), S["heads"])
        torch.cuda.synchronize()
        self._compare(t, S, o_dev, o_ref, (pre_codes, pre_scales, inputs))
        self.rep.head_steps += len(S["heads"])

    def _compare(self, t, S, o_dev, o_ref, pre):
        w = self.w
        cg = self._gather(self.gpu.codes, S["ci_d"])
        sg = self._gather(self.gpu.scales, S["si_d"])
        cr, sr = self.codes[S["ci"]], self.scales[S["si"]]
        self.rep.elements += len(S["heads"]) * w.dv * w.dk
        if not np.array_equal(sg.view(np.uint32), sr.view(np.uint32)):
            bad = np.nonzero(sg.view(np.uint32) != sr.view(np.uint32))[0]
            raise ParityError(f"step {t}: {bad.size} scales differ, first in head "
                              f"{S['heads'][bad[0] // self.n_scales]}")
        if not np.array_equal(cg, cr):
            self._exempt_heads(t, S, cg, cr, pre)
        if o_dev is not None:
            og = self._gather(o_dev, S["oi_d"])
            orf = o_ref[S["oi"]]
            err = np.abs(og.astype(np.float64) - orf.astype(np.float64))
            self.rep.max_o_err = max(self.rep.max_o_err, float(err.max()))
            ok = err <= ATOL + RTOL * np.abs(orf.astype(np.float64))
            if not np.all(ok):
                i = int(np.argmin(ok))
                raise ParityError(f"step {t}: o differs in head {S['heads'][i // w.dv]} row "
                                  f"{i % w.dv}: gpu {og[i]} ref {orf[i]}")
        check_rate(self.rep.exempt, self.rep.elements, f"step {t}")

    def _exempt_heads(self, t, S, cg, cr, pre):
        """Per differing head: recompute the reference step with threshold
        distances and apply the exemption rule; then re-sync the GPU head."""
        w = self.w
        pos = 0
        for bh in S["heads"]:
            n = int(self.hbytes[bh % w.H])
            g, r = cg[pos:pos + n], cr[pos:pos + n]
            if not np.array_equal(g, r):
                b, h = divmod(int(bh), w.H)
                td = self._tdist(t, S, pos, bh, pre)
                bad = classify(_decode(g, self.bb[h], w.dv, w.dk),
                               _decode(r, self.bb[h], w.dv, w.dk), td, f"step {t} head {(b, h)}")
                self.rep.exempt += len(bad)
                if self.rep.first_exempt_step < 0:
                    self.rep.first_exempt_step = t
                off = self._off(bh)
                self.gpu.codes[off:off + n] = torch.from_numpy(r.copy()).cuda()
            pos += n

    def _tdist(self, t, S, pos, bh, pre):
        w = self.w
        b, h = divmod(int(bh), w.H)
        ci = np.nonzero(S["heads"] == bh)[0][0]
        n = int(self.hbytes[h])
        if isinstance(pre[0], str):  # the import: quantize the reference FP32 state again
            hs = w.dv * w.dk
            S_head = pre[1][int(bh) * hs:(int(bh) + 1) * hs].reshape(w.dv, w.dk)
            return oracle.head_quantize(self.ocfg, b, h, self.bb[h], S_head, 0, want_tdist=True)[2]
        pre_codes, pre_scales, (q, k, v, alpha, beta) = pre
        codes = pre_codes[pos:pos + n].copy()
        scales = pre_scales[ci * self.n_scales:(ci + 1) * self.n_scales].copy()
        a = alpha[b, h] if w.mixer in (W.GLA, W.KDA) else np.float32([alpha[b, h]])
        bt = 0.0 if beta is None else float(beta[b, h])
        _, _, td = oracle.head_step(self.ocfg, b, h, self.bb[h], codes, scales, q[b, h], k[b, h],
                                    v[b, h], a, bt, t, want_tdist=True)
        return td

    def _final_check(self, pre_q):
        """Export and readout of the tracked heads after the last step."""
        w = self.w
        S = self.S_tracked
        n = w.B * w.H * w.dv * w.dk
        Sd = torch.empty(n, dtype=torch.float32, device="cuda")
        self.gpu.store_fp32(Sd)
        o = torch.empty(w.B * w.H * w.dv, dtype=torch.float32, device="cuda")
        self.gpu.readout(_dev(pre_q), o)
        torch.cuda.synchronize()
        hs = w.dv * w.dk
        sidx = (S["heads"][:, None] * hs + np.arange(hs)[None, :]).ravel()
        Sg = (Sd if S["full"] else Sd.index_select(0, torch.from_numpy(sidx).cuda())).cpu().numpy()
        og = self._gather(o, S["oi_d"])
        for i, bh in enumerate(S["heads"]):
            b, h = divmod(int(bh), w.H)
            off, nb = self._off(bh), int(self.hbytes[h])
            codes = self.codes[off:off + nb]
            scales = self.scales[bh * self.n_scales:(bh + 1) * self.n_scales]
            Sr = oracle.head_dequantize(self.ocfg, self.bb[h], codes, scales).ravel()
            if not np.array_equal(Sg[i * hs:(i + 1) * hs], Sr):
                raise ParityError(f"export differs at head {(b, h)}")
            orr = oracle.head_readout(self.ocfg, self.bb[h], codes, scales, pre_q[b, h])
            og_h = og[i * w.dv:(i + 1) * w.dv].astype(np.float64)
            if not np.all(np.abs(og_h - orr) <= ATOL + RTOL * np.abs(orr.astype(np.float64))):
                raise ParityError(f"readout differs at head {(b, h)}")


def sample_heads(w: W.Workload, n: int, seed: int) -> np.ndarray:
    """A seeded sample of n heads (b*H + h) that includes the first and last
    head and every head index h at least once."""
    rng = np.random.default_rng(seed)
    total = w.B * w.H
    pick = set(rng.choice(total, min(n, total), replace=False).tolist())
    pick |= {0, total - 1}
    pick |= {int(rng.integers(0, w.B)) * w.H + h for h in range(w.H)}
    return np.array(sorted(pick), np.int64)
