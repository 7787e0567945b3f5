#!/usr/bin/env python3
"""Benchmark of the quantized recurrent-state decode step on one MI355X.

A step is one qstate_step over the whole batch (every head: dequantize,
update, readout, requantize).  The headline workload is the Gated DeltaNet
decode at B=256, H=32, dk=dv=128, INT4 state with INT8 for the slowest-
decaying heads, group 32, stochastic rounding.

Cold protocol (the reported value): steps rotate over `--states` independent
state instances (one per layer, each with its own stochastic-rounding key) so
that the per-step working set is far larger than the 256 MB Infinity Cache,
as in a model whose layers each hold a state; step inputs come from a pool of
pre-generated batches already resident in HBM.  The hot number (one state,
cache-resident) is reported beside it.

Prints one JSON line.  The CPU reference is timed on a bounded sample of
heads for the cpu_baseline figure.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-state decode steps/s and HBM GB/s (% of peak) at B=256, INT8/INT4"
HBM_PEAK_GBPS = 8000.0
# Vector ALU issue peak, in T lane-instructions/s: the published FP32 vector
# rate (157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 FMA lanes per clock x 2 flops
# at 2.4 GHz), i.e. one wave64 FP32 instruction per SIMD every 2 clocks.
# Integer, conversion, SDWA/DPP and three-operand min/max forms take longer
# per instruction, so a real mix stays below this figure even when issue-bound.
VALU_PEAK_TLANES = 256 * 4 * 32 * 2.4e9 / 1e12
ROUNDING_NAMES = {0: "RTN", 1: "SR", 2: "BDR"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_unit(w) -> str:
    """The translation unit holding the step kernels of workload w."""
    if w.window:
        return f"qstate_window_dk{w.dk}_w{w.window}.hip"
    if w.axis:
        return f"qstate_key_dk{w.dk}.hip"
    return f"qstate_value_dk{w.dk}.hip"


def kernel_source_hash(w) -> str:
    """The source hash of w's step kernels (their unit, the headers it
    includes, the launch code and the compile flags): stored profiler counts
    apply only while it is unchanged."""
    from bit_recurrent_state_amd import build
    return build.unit_hash(kernel_unit(w))


def traffic_key(w) -> str:
    """The record key of w's profiler counts: workload, rounding, axis, window
    and bypass, plus the batch and width policy where they differ from the
    workload's own (records are per shape and width mix)."""
    import workloads as W
    key = f"{w.name}|{ROUNDING_NAMES[w.rounding]}|{'key' if w.axis else 'value'}-axis"
    key += f"|window{w.window}" if w.window else ""
    key += "|lrb" if w.window_merge else ""
    base = W.WORKLOADS[w.wid]
    key += f"|B{w.B}" if w.B != base.B else ""
    key += f"|bits={w.bits_policy}" if w.bits_policy != base.bits_policy else ""
    return key


def measured_traffic(w):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts of this workload, rounding and group axis (scaled by the same
    counters on the library's 2 GiB in-place read-modify-write kernel); None
    when they were not taken or the kernel source changed since."""
    try:
        import json as _j
        t = _j.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(traffic_key(w))
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash(w):
        return None
    return e["hbm_bytes_per_launch"]


def measured_clock(w):
    """Shader clock (GHz) of this workload's step kernel from the committed
    rocprofv3 SQ_BUSY_CU_CYCLES record (median over dispatches); None when it
    was not taken or the kernel source changed since."""
    try:
        import json as _j
        t = _j.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(traffic_key(w))
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash(w):
        return None
    return e.get("shader_clock_ghz")


def measured_valu(w):
    """VALU wave-instructions per launch from the committed rocprofv3
    SQ_INSTS_VALU count of this workload's step kernel; None when it was not
    taken or the kernel source changed since."""
    try:
        import json as _j
        t = _j.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(traffic_key(w))
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash(w):
        return None
    return e.get("valu_wave_insts_per_launch")


def gate_bytes(w) -> int:
    """alpha (one per head, or one per key channel for GLA and KDA) and beta
    (absent for GLA)."""
    import workloads as W
    alpha = 4 * w.dk if w.mixer in (W.GLA, W.KDA) else 4
    return alpha + (0 if w.mixer == W.GLA else 4)


def block_bits(w, Q) -> np.ndarray:
    """Widths per head and 16-column block [H][dk/16] from the workload's
    decay-based policy (per head, or per group of G key channels)."""
    import workloads as W
    nb = w.dk // 16
    if w.bits_policy == "channel_half":
        ret = W.group_retention(w)
        return np.stack([np.repeat(Q.qstate_bits_by_decay(ret[h], 1, 0.5), w.G // 16)
                         for h in range(w.H)]).astype(np.uint8)
    policy = {"alpha_gt_0.99": (0, 0.99), "rank_half": (1, 0.5)}.get(w.bits_policy)
    hb = (Q.qstate_bits_by_decay(W.head_retention(w), *policy) if policy
          else np.full(w.H, 4 if w.bits_policy == "int4" else 8, np.uint8))
    return np.repeat(hb[:, None], nb, axis=1).astype(np.uint8)


def algorithmic_bytes(w, bb) -> int:
    """Bytes one step must move: each head's codes and scales read and written
    once, q, k, v, o, and the gates (alpha per head or per key channel, beta).
    bb: widths per head and 16-column block."""
    per_b = 0
    for h in range(w.H):
        state = w.dv * int(np.sum(2 * bb[h].astype(np.int64))) + w.dv * w.dk // w.G * 4
        if w.window:  # pure-write window: a codes read + the new pair's, keys and scales
            W = w.window
            per_b += w.dv * W + w.dv + 2 * (W * w.dk + 8 * W)
            if w.window_merge:  # bypass: a merge step (1 in W) rewrites every a code of a row
                per_b += w.dv * (W - 1) / W
        io = 4 * (2 * w.dk + 2 * w.dv)
        per_b += 2 * state + io + gate_bytes(w)
    return int(round(per_b * w.B))


def fp32_bytes(w) -> int:
    per_head = 2 * w.dv * w.dk * 4 + 4 * (2 * w.dk + 2 * w.dv) + gate_bytes(w)
    return per_head * w.B * w.H


def fp32_accuracy(w, hb, Q, torch, batch: int = 8, checkpoints=(1, 64, 256, 1024)):
    """Readouts of the quantized state against an FP32-state run of the same
    recurrence and inputs: rel-L2 of o over all heads at the checkpoints.
    Heads are independent, so a batch of `batch` rows of the workload's heads
    (same per-head widths, inputs drawn fresh every step) stands for B."""
    import workloads as W
    wb = w.scaled(B=batch)
    n = wb.B * wb.H

    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

    uniform = bool(np.all(hb == hb[:, :1]))
    f = Q.QState(Q.Config(wb.B, wb.H, wb.dk, wb.dv, 16, wb.mixer, 0, True, None, 0, 0))
    f.load_fp32(torch.zeros(n * wb.dv * wb.dk, device="cuda"))
    for t in range(wb.warmup):
        f.step(*map(dev, W.step_inputs(wb, t)))
    S = torch.empty(n * wb.dv * wb.dk, device="cuda")
    f.store_fp32(S)
    qs = Q.QState(Q.Config(wb.B, wb.H, wb.dk, wb.dv, wb.G, wb.mixer, wb.rounding, False,
                           hb[:, 0].tolist() if uniform else None, 0, 0, wb.axis,
                           None if uniform else hb.tolist(), wb.window, wb.window_merge,
                           wb.lrb_threshold))
    qs.load_fp32(S)
    o_q = torch.empty(n * wb.dv, device="cuda")
    o_f = torch.empty_like(o_q)
    out = {}
    for t in range(1, max(checkpoints) + 1):
        inp = tuple(map(dev, W.step_inputs(wb, wb.warmup + t - 1)))
        qs.step(*inp, o_q)
        f.step(*inp, o_f)
        if t in checkpoints:
            out[str(t)] = float(torch.linalg.vector_norm(o_q - o_f) / torch.linalg.vector_norm(o_f))
    qs.close()
    f.close()
    return {"rel_l2_o": out, "batch": wb.B, "heads": n,
            "note": "quantized vs FP32 state, same warm-up state and inputs"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, hb, seconds: float, single_seconds: float):
    """The CPU reference on a sample of heads: one thread alone, then one
    thread per host core (every core of the affinity mask).  Heads are
    independent, so each thread steps its own heads; head-steps per second,
    scaled to steps/s of the workload.  Each thread's heads (quantized state
    and argument pointers) are prepared before the clock starts; the timed
    loop only calls the reference's C entry point."""
    import ctypes
    import threading

    import oracle
    import workloads as W

    rng = np.random.default_rng(0)
    c = oracle.cfg(w.B, w.H, w.dk, w.dv, w.G, w.mixer, w.rounding, 0, 0, w.axis, w.window,
                   w.window_merge, w.lrb_threshold)
    q, k, v, alpha, beta = W.step_inputs(w, 0)
    S0 = rng.standard_normal((w.dv, w.dk)).astype(np.float32)
    L = oracle.lib()
    P = ctypes.c_void_p
    per_thread = 4

    def prepare(n_threads):
        sets = []
        for _ in range(n_threads):
            mine = []
            for b, h in zip(rng.integers(0, w.B, per_thread), rng.integers(0, w.H, per_thread)):
                b, h = int(b), int(h)
                codes, scales, _ = oracle.head_quantize(c, b, h, hb[h], S0, 0)
                a = alpha[b, h] if w.mixer in (W.GLA, W.KDA) else np.float32([alpha[b, h]])
                keep = [np.ascontiguousarray(x, np.float32) for x in (q[b, h], k[b, h], v[b, h], a)]
                keep += [np.ascontiguousarray(hb[h], np.uint8), codes, scales,
                         np.zeros(max(oracle.window_bytes(c), 16), np.uint8)]
                mine.append((b, h, keep, [P(x.ctypes.data) for x in keep],
                             0.0 if beta is None else float(beta[b, h])))
            sets.append(mine)
        return sets

    def run(n_threads, secs):
        sets = prepare(n_threads)
        counts = [0] * n_threads
        start = threading.Barrier(n_threads + 1)

        def work(wi, deadline_box):
            mine = sets[wi]
            start.wait()
            deadline = deadline_box[0]
            n = 0
            while time.perf_counter() < deadline:
                b, h, _keep, ptr, bt = mine[n % len(mine)]
                pq, pk, pv, pa, pbb, pc, ps, pw = ptr
                if w.window:
                    L.oracle_head_step_pw(ctypes.byref(c), b, h, pbb, pc, ps, pw, pq, pk, pv, pa,
                                          bt, None, 1 + n, None, None)
                else:
                    L.oracle_head_step(ctypes.byref(c), b, h, pbb, pc, ps, pq, pk, pv, pa, bt,
                                       None, 1 + n, None, None)
                n += 1
            counts[wi] = n

        box = [0.0]
        threads = [threading.Thread(target=work, args=(i, box)) for i in range(n_threads)]
        for t in threads:
            t.start()
        box[0] = time.perf_counter() + secs
        t0 = time.perf_counter()
        start.wait()
        for t in threads:
            t.join()
        dt = time.perf_counter() - t0
        return sum(counts), dt

    n1, dt1 = run(1, single_seconds)
    cores = host_cores()
    n, dt = run(cores, seconds)
    heads = w.B * w.H
    return {
        "value": n / dt / heads,
        "unit": "steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n} head-steps of the same workload ({w.dv}x{w.dk} heads, "
                  f"{ROUNDING_NAMES[w.rounding]}) in {dt:.1f} s on {cores} host threads "
                  f"(every core of the affinity mask, disjoint heads; {dt * cores:.0f} "
                  f"CPU-seconds), scaled by the {heads} heads of one step",
        "single_thread": {"value": n1 / dt1 / heads, "unit": "steps/s", "cores": 1,
                          "sample": f"{n1} head-steps in {dt1:.1f} s on one thread"},
        "cpu_model": cpu_model(),
    }


def input_pool(w, torch, first_t, min_bytes, layer=0):
    """Pre-generated input batches (drawn on host threads, then copied to the
    device) whose total size exceeds min_bytes, so that q, k, v and the gates
    stream from HBM rather than from the 256 MB Infinity Cache."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads as W
    one = W.step_inputs(w, first_t, 0, layer)
    per = sum(x.nbytes for x in one if x is not None) + 4 * w.B * w.H * w.dv  # + o
    n = max(2, int(np.ceil(min_bytes / per)))
    with ThreadPoolExecutor(max_workers=min(16, host_cores())) as ex:
        batches = list(ex.map(lambda t: W.step_inputs(w, t, 0, layer),
                              range(first_t, first_t + n)))

    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

    pool = [tuple(map(dev, b)) for b in batches]
    return pool, n * per


def warm_state(w, Q, torch, layer=0):
    """The workload's FP32 warm-up on the GPU from zero: the state every
    instance is imported from."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads as W

    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

    f = Q.QState(Q.Config(w.B, w.H, w.dk, w.dv, 16, w.mixer, 0, True, None, 0, layer))
    f.load_fp32(torch.zeros(w.B * w.H * w.dv * w.dk, device="cuda"))
    with ThreadPoolExecutor(max_workers=min(16, host_cores())) as ex:
        for inp in ex.map(lambda t: W.step_inputs(w, t, 0, layer), range(w.warmup)):
            f.step(*map(dev, inp))
    S = torch.empty(w.B * w.H * w.dv * w.dk, device="cuda")
    f.store_fp32(S)
    f.close()
    return S


def qconfig(Q, w, hb, layer):
    uniform = bool(np.all(hb == hb[:, :1]))
    return Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, w.rounding, False,
                    hb[:, 0].tolist() if uniform else None, 0, layer, w.axis,
                    None if uniform else hb.tolist(), w.window, w.window_merge, w.lrb_threshold)


def timed(torch, launches, steps, warm):
    """ms per step: `launches` is a list of steps, each a list of (state,
    inputs, o) launches; steps run round-robin over the list on torch's
    current stream (the one the library launches on), timed with HIP events
    on that stream."""
    stream = torch.cuda.current_stream()
    for i in range(warm):
        for st, inp, o in launches[i % len(launches)]:
            st.step(*inp, o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        for st, inp, o in launches[i % len(launches)]:
            st.step(*inp, o)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def roofline(nbytes, ms):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": nbytes}


def measure_workload(w, Q, torch, steps, warm, min_state_bytes=2**30, min_pool_bytes=320e6):
    """Cold protocol for one single-layer workload: >= 1 GiB of independent
    state instances (one per layer key), a > 320 MB input pool."""
    hb = block_bits(w, Q)
    cb, sb = Q.qstate_state_bytes(qconfig(Q, w, hb, 0))
    n_states = max(2, int(np.ceil(min_state_bytes / (cb + sb))))
    S = warm_state(w, Q, torch)
    states = []
    for layer in range(n_states):
        st = Q.QState(qconfig(Q, w, hb, layer))
        st.load_fp32(S)
        states.append(st)
    del S
    pool, pool_bytes = input_pool(w, torch, w.warmup, min_pool_bytes)
    o = torch.empty(w.B * w.H * w.dv, device="cuda")
    launches = [[(states[i % n_states], pool[i % len(pool)], o)]
                for i in range(n_states * len(pool))]
    ms = timed(torch, launches, steps, warm)
    nbytes = algorithmic_bytes(w, hb)
    for st in states:
        st.close()
    del states, pool, launches
    torch.cuda.empty_cache()
    return {"workload": w.name, "rounding": ROUNDING_NAMES[w.rounding], "B": w.B, "H": w.H,
            "ms_per_step": ms, "steps_per_s": 1e3 / ms, "roofline": roofline(nbytes, ms),
            "state_instances": n_states, "state_MB_each": round((cb + sb) / 1e6, 1),
            "input_pool_MB": round(pool_bytes / 1e6, 1), "steps": steps}


def measure_layer_stack(w, Q, torch, steps, warm, min_pool_bytes=320e6):
    """The Mamba2-style stack as one step: w.layers independent states (layer
    keys 0..L-1, widths by each layer's decay ranking), one launch each per
    step.  Every layer is imported from the same FP32 warm-up (layer 0's
    inputs); the input pool is shared by the layers."""
    import workloads as W
    S = warm_state(w, Q, torch)
    states, nbytes, sbytes = [], 0, 0
    for layer in range(w.layers):
        rule = {"rank_half": (1, 0.5), "alpha_gt_0.99": (0, 0.99)}[w.bits_policy]
        hb1 = Q.qstate_bits_by_decay(W.head_retention(w, 0, layer), *rule)
        hb = np.repeat(hb1[:, None], w.dk // 16, axis=1).astype(np.uint8)
        st = Q.QState(qconfig(Q, w, hb, layer))
        st.load_fp32(S)
        states.append(st)
        nbytes += algorithmic_bytes(w, hb)
        cb, sb = Q.qstate_state_bytes(qconfig(Q, w, hb, layer))
        sbytes += cb + sb
    del S
    pool, pool_bytes = input_pool(w, torch, w.warmup, min_pool_bytes)
    o = torch.empty(w.B * w.H * w.dv, device="cuda")
    launches = [[(states[l], pool[(i * w.layers + l) % len(pool)], o) for l in range(w.layers)]
                for i in range(len(pool))]
    ms = timed(torch, launches, steps, warm)
    for st in states:
        st.close()
    del states, pool, launches
    torch.cuda.empty_cache()
    rf = roofline(nbytes, ms)
    return {"workload": w.name, "rounding": ROUNDING_NAMES[w.rounding], "B": w.B, "H": w.H,
            "layers": w.layers, "ms_per_step": ms, "steps_per_s": 1e3 / ms,
            "ms_per_layer_launch": ms / w.layers, "roofline": rf,
            "state_MB_all_layers": round(sbytes / 1e6, 1),
            "input_pool_MB": round(pool_bytes / 1e6, 1), "steps": steps,
            "note": "one step = one launch per layer; layers imported from one FP32 warm-up"}


def ceilings(Q, torch, nbytes=2**31, reps=20):
    """The library's own bandwidth-ceiling kernels on a 2 GiB buffer (8x the
    Infinity Cache): streaming copy and in-place read-modify-write, with and
    without the non-temporal hint; GB/s counts bytes read plus written."""
    import ctypes

    from bit_recurrent_state_amd._lib import check, lib
    L = lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    out = {}
    for name, fn in (("copy", lambda nt: L.qstate_ceiling_copy(ctypes.c_void_p(a.data_ptr()),
                                                             ctypes.c_void_p(b.data_ptr()),
                                                             nbytes, nt, sp)),
                     ("rmw", lambda nt: L.qstate_ceiling_rmw(ctypes.c_void_p(a.data_ptr()),
                                                           nbytes, 0x5A5A5A5A, nt, sp))):
        for nt in (1, 0):
            for _ in range(3):
                check(f"qstate_ceiling_{name}", fn(nt))
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn(nt)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[f"{name}{'_nt' if nt else ''}_gbps"] = 2 * nbytes / (ms * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["kernel"] = "qstate_ceiling_copy / qstate_ceiling_rmw, 2 GiB, 16 B per lane access"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--rounding", type=int, default=None, help="override: 0 RTN, 1 SR, 2 BDR")
    ap.add_argument("--axis", type=int, default=0,
                    help="scale groups: 0 value axis (default), 1 key axis")
    ap.add_argument("--window", type=int, default=0,
                    help="pure-write window length (0 = none, 4, 8, 16)")
    ap.add_argument("--lrb", type=float, default=None, metavar="THRESHOLD",
                    help="low-rank bypass with this merge threshold (needs --window)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch B")
    ap.add_argument("--bits", choices=["int4", "int8"], default=None,
                    help="override the per-head width policy: every head INT4 or INT8")
    ap.add_argument("--states", type=int, default=0, help="state instances (0: >= 1 GiB)")
    ap.add_argument("--pool-mb", type=float, default=320.0,
                    help="pre-generated input batches of at least this many MB")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="wall seconds of the CPU-reference sample on every host core")
    ap.add_argument("--cpu-single-seconds", type=float, default=7.0,
                    help="wall seconds of the single-thread CPU-reference sample")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads, hot, FP32-state and ceiling figures")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the ceiling kernels even with --no-extras (their known "
                         "byte counts calibrate profiler traffic counters in the same run)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU (heads shard across GPUs with no exchange); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import workloads as W
    from bit_recurrent_state_amd import qstate as Q

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    w = W.WORKLOADS[args.workload]
    if args.rounding is not None:
        w = w.scaled(rounding=args.rounding)
    w = w.scaled(axis=args.axis, window=args.window)
    if args.batch:
        w = w.scaled(B=args.batch)
    if args.bits:
        w = w.scaled(bits_policy=args.bits)
    if args.lrb is not None:
        if not args.window:
            print(json.dumps({"error": "--lrb needs --window"}))
            sys.exit(2)
        w = w.scaled(window_merge=1, lrb_threshold=args.lrb)
    hb = block_bits(w, Q)  # [H][dk/16]
    uniform = bool(np.all(hb == hb[:, :1]))
    nbytes = algorithmic_bytes(w, hb)

    cb, sb = Q.qstate_state_bytes(qconfig(Q, w, hb, 0))
    n_states = args.states or max(2, int(np.ceil(1.0 * 2**30 / (cb + sb))))
    S = warm_state(w, Q, torch)
    states = []
    for layer in range(n_states):
        st = Q.QState(qconfig(Q, w, hb, layer))
        st.load_fp32(S)
        states.append(st)
    del S
    pool, pool_bytes = input_pool(w, torch, w.warmup, args.pool_mb * 1e6)
    o = torch.empty(w.B * w.H * w.dv, device="cuda")
    torch.cuda.synchronize()
    launches = [[(states[i % n_states], pool[i % len(pool)], o)]
                for i in range(n_states * len(pool))]

    ms = timed(torch, launches, args.steps, args.warmup)
    # the same launches again as 5 repetitions, for the spread (the value
    # above stays the one timed region of exactly --steps steps)
    reps = [timed(torch, launches, max(1, args.steps // 5), 0) for _ in range(5)]
    rf = roofline(nbytes, ms)
    rf["traffic"] = measured_traffic(w)
    gbps = rf["achieved"]
    result = {
        "metric": METRIC,
        "value": 1e3 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv, "group": w.G,
            "state_bits": ({str(b): int((hb[:, 0] == b).sum()) for b in sorted(set(hb[:, 0].tolist()))}
                           if uniform else
                           {f"{b}-bit 16-channel blocks": int((hb == b).sum())
                            for b in sorted(set(hb.ravel().tolist()))}),
            "rounding": ROUNDING_NAMES[w.rounding],
            "group_axis": "key" if w.axis else "value", "window": w.window,
            **({"low_rank_bypass_threshold": w.lrb_threshold} if w.window_merge else {}),
            "state_instances": n_states,
            "state_MB_each": round((cb + sb) / 1e6, 1),
            "input_pool_MB": round(pool_bytes / 1e6, 1), "input_batches": len(pool),
        },
        "hbm_gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "repetitions": {"ms_per_step": reps, "median_ms_per_step": float(np.median(reps)),
                        "steps_each": max(1, args.steps // 5)},
        "roofline": rf,
    }
    # The same launches against the vector-ALU issue rate (the INT4 + SR path
    # is bound there): measured VALU instructions x 64 lanes / launch time.
    vi = measured_valu(w)
    if vi:
        tl = vi * 64 / (ms * 1e-3) / 1e12
        result["valu_roofline"] = {"bound": "alu", "achieved": tl, "peak": VALU_PEAK_TLANES,
                                   "unit": "T lane-instructions/s", "frac": tl / VALU_PEAK_TLANES,
                                   "wave_insts_per_launch": vi,
                                   "lane_insts_per_state_element": vi * 64 / (w.B * w.H * w.dv * w.dk)}
        clk = measured_clock(w)
        if clk:  # the same issue rate at the clock the chip held during the step
            result["valu_roofline"]["measured_clock_ghz"] = clk
            result["valu_roofline"]["frac_at_measured_clock"] = tl / (VALU_PEAK_TLANES * clk / 2.4)

    if not args.no_extras:
        result["accuracy_vs_fp32_state"] = fp32_accuracy(w, hb, Q, torch)
        ms_hot = timed(torch, [[(states[0], pool[i % len(pool)], o)] for i in range(len(pool))],
                       args.steps, args.warmup)
        result["hot_single_state"] = {"ms_per_step": ms_hot, "steps_per_s": 1e3 / ms_hot,
                                      "effective_gbps": nbytes / (ms_hot * 1e-3) / 1e9}
    for st in states:
        st.close()
    del states, pool, launches
    torch.cuda.empty_cache()

    if not args.no_extras:
        steps_x = max(args.steps, 200)
        # the other B = 256 workload (GLA, INT8, group 64), both roundings, and
        # the 24-layer Mamba2-style stack as one step
        others = {}
        for rnd in (W.RTN, W.SR):
            wx = W.WORKLOADS[3].scaled(rounding=rnd)
            others[f"{wx.name}_{ROUNDING_NAMES[rnd].lower()}"] = measure_workload(
                wx, Q, torch, steps_x, 20)
        w4 = W.WORKLOADS[4]
        others[w4.name] = measure_layer_stack(w4, Q, torch, max(20, steps_x // 10), 3)
        result["other_workloads"] = others
        # FP32-state baseline kernel, same protocol
        fb = fp32_bytes(w)
        n_f = max(2, int(np.ceil(1.0 * 2**30 / (fb / 2))))
        fstates = []
        for layer in range(n_f):
            fs = Q.QState(Q.Config(w.B, w.H, w.dk, w.dv, 16, w.mixer, 0, True, None, 0, layer))
            fs.load_fp32(torch.zeros(w.B * w.H * w.dv * w.dk, device="cuda"))
            fstates.append(fs)
        fpool, _ = input_pool(w, torch, w.warmup, 0)
        of = torch.empty(w.B * w.H * w.dv, device="cuda")
        ms_f = timed(torch, [[(fstates[i % n_f], fpool[i % len(fpool)], of)]
                             for i in range(n_f * len(fpool))], max(200, args.steps // 4), 10)
        result["fp32_state_baseline"] = {
            "ms_per_step": ms_f, "steps_per_s": 1e3 / ms_f, "state_instances": n_f,
            "gbps": fb / (ms_f * 1e-3) / 1e9, "speedup_of_quantized": ms_f / ms}
        for fs in fstates:
            fs.close()
        del fstates, fpool
        torch.cuda.empty_cache()
    if not args.no_extras or args.ceilings:
        cl = ceilings(Q, torch)
        result["ceiling"] = cl
        result["hbm_frac_of_rmw_ceiling"] = gbps / max(cl["rmw_nt_gbps"], cl["rmw_gbps"])

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, hb, args.cpu_seconds, args.cpu_single_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
