"""GPU parity: the HIP library (through its C ABI) against the CPU reference.

Every case runs the whole workload on both sides from the same seeded
inputs; see tests/parity.py for the comparison contract."""

import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

if gpu_available():
    import torch

    import oracle
    import workloads as W
    from bit_recurrent_state_amd import qstate as Q
    from parity import Run, log
else:  # keep collection working on CPU-only hosts
    import workloads as W


def _run(w, steps, rounding=None, heads=None, seed=0, layer=0, hb=None):
    r = Run(w, rounding, seed, layer, heads, head_bits_override=hb)
    log(f"[case] {w.name} B={w.B} H={w.H} dk={w.dk} dv={w.dv} G={w.G} axis={w.axis} mixer={w.mixer} "
        f"rounding={r.rounding} bits={sorted(set(r.hb.tolist()))} warmup={w.warmup} "
        f"steps={steps} heads={len(r.heads)} seed={seed} layer={layer}")
    r.warmup_and_import()
    for _ in range(steps):
        r.step()
    r.dequant_check()
    r.close()
    log(f"[done] steps={r.rep.steps} elements={r.rep.elements} exempt={r.rep.exempt} "
        f"max_o_err={r.rep.max_o_err:.3g}")
    return r.rep


def test_config0_every_step_every_head():
    rep = _run(W.WORKLOADS[0], W.WORKLOADS[0].steps)
    assert rep.exempt == 0


def test_config1_int8_sr_every_head():
    _run(W.WORKLOADS[1].scaled(B=4), 24)


def test_config2_int4_int8_mix_every_head():
    w = W.WORKLOADS[2].scaled(B=2)
    from parity import head_bits
    hb = head_bits(w)
    assert 4 in hb and 8 in hb  # the decay rule gives a real mix
    _run(w, 12)


@pytest.mark.parametrize("rounding", [W.RTN, W.SR])
def test_config3_gla_every_head(rounding):
    _run(W.WORKLOADS[3].scaled(B=3), 10, rounding=rounding)


@pytest.mark.parametrize("rounding", [W.RTN, W.SR])
def test_kda_every_head(rounding):
    _run(W.WORKLOADS[5].scaled(B=3), 10, rounding=rounding)


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_bdr_every_head(wid):
    """Bounded directional rounding on every recurrence, mixed bits included."""
    _run(W.WORKLOADS[wid].scaled(B=2), 10, rounding=W.BDR)


@pytest.mark.parametrize("mixer,G", [(W.GDN, 128), (W.GDN, 16), (W.SCALAR, 128)])
def test_bdr_group_sizes(mixer, G):
    """BDR with mostly INT4 heads at the group sizes the workloads do not use
    (one group spanning four lanes, two groups per lane): persistent and
    sliced steps alike."""
    w = W.Workload(90 + 10 * mixer + G // 16, f"bdr_m{mixer}_g{G}", mixer, 2, 4, 128, 128, G, 6,
                   12, W.BDR, "int8")
    _run(w, 12, hb=np.array([4, 4, 8, 4], np.uint8), seed=23)


def test_bdr_full_size_sampled_heads():
    w = W.WORKLOADS[2]
    rng = np.random.default_rng(12)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    _run(w, 2, rounding=W.BDR, heads=sorted((i // w.H, i % w.H) for i in idx))


KEY_AXIS_RUNS = [(2, W.SR), (3, W.RTN), (3, W.BDR), (4, W.SR), (5, W.SR), (1, W.BDR)]


@pytest.mark.parametrize("wid,rounding", KEY_AXIS_RUNS)
def test_key_axis_every_head(wid, rounding):
    """Key-axis scale groups (G value rows of one key column) on every
    recurrence and rounding, mixed bits included."""
    _run(W.WORKLOADS[wid].scaled(B=2, axis=1), 8, rounding=rounding)


# key-axis block shapes: several groups per wave, one group over 2, 4 and 8
# waves, groups longer than dk, ragged dv (a partial last block)
KEY_RAGGED = [
    (W.GDN, W.SR, 64, 48, 16, [8, 4, 4]),
    (W.GLA, W.RTN, 128, 80, 16, [4, 8]),
    (W.KDA, W.BDR, 128, 128, 128, [8, 4]),
    (W.SCALAR, W.SR, 64, 128, 128, [4, 8]),
    (W.GDN, W.RTN, 256, 256, 128, [8]),
    (W.GDN, W.BDR, 256, 96, 32, [4, 8]),
]


@pytest.mark.parametrize("mixer,rounding,dk,dv,G,bits", KEY_RAGGED)
def test_key_axis_shapes(mixer, rounding, dk, dv, G, bits):
    w = W.Workload(85 + mixer, f"key_m{mixer}_dk{dk}_dv{dv}_g{G}", mixer, 3, len(bits), dk, dv, G,
                   5, 3, rounding, "int8", axis=1)
    _run(w, 5, hb=np.array(bits, np.uint8), seed=11)


def test_key_axis_full_size_sampled_heads():
    w = W.WORKLOADS[2].scaled(axis=1)
    rng = np.random.default_rng(21)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    _run(w, 2, heads=sorted((i // w.H, i % w.H) for i in idx))


@pytest.mark.parametrize("rounding,axis", [(W.SR, 0), (W.RTN, 0), (W.BDR, 0), (W.SR, 1)])
def test_channel_bits_every_head(rounding, axis):
    """Per-channel widths (INT8 for the slower half of each head's 32-channel
    groups, INT4 for the rest) on every head, both group axes."""
    w = W.WORKLOADS[6].scaled(B=2, axis=axis)
    from parity import block_bits
    bb = block_bits(w)
    assert np.any(bb == 8) and np.any(bb == 4) and not np.all(bb == bb[:, :1])
    _run(w, 8, rounding=rounding)


# mixed widths per 16-column block inside a head, ragged rows, every dk
CHANNEL_RAGGED = [
    (W.GDN, W.SR, 0, 64, 37, 16, [[8, 4, 4, 8], [4, 8, 8, 4], [4, 4, 4, 4]]),
    (W.KDA, W.BDR, 0, 256, 45, 32, [[8, 8, 4, 4] * 4, [4, 4, 8, 8, 8, 8, 4, 4] * 2]),
    (W.SCALAR, W.RTN, 0, 128, 70, 64, [[8] * 4 + [4] * 4, [8] * 8]),
    (W.GLA, W.SR, 1, 128, 64, 32, [[8, 4, 8, 4, 4, 8, 4, 8], [4] * 8]),
    (W.GDN, W.BDR, 1, 64, 128, 128, [[4, 8, 4, 8], [8, 8, 4, 4]]),
]


@pytest.mark.parametrize("mixer,rounding,axis,dk,dv,G,bits", CHANNEL_RAGGED)
def test_channel_bits_shapes(mixer, rounding, axis, dk, dv, G, bits):
    w = W.Workload(75 + mixer, f"chan_m{mixer}_dk{dk}_dv{dv}_g{G}_a{axis}", mixer, 3, len(bits),
                   dk, dv, G, 5, 3, rounding, "int8", axis=axis)
    _run(w, 5, hb=np.array(bits, np.uint8), seed=13)


def test_channel_bits_full_size_sampled_heads():
    w = W.WORKLOADS[6]
    rng = np.random.default_rng(31)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    _run(w, 2, heads=sorted((i // w.H, i % w.H) for i in idx))


WINDOW_RUNS = [(2, W.SR, 8), (3, W.RTN, 4), (5, W.BDR, 16), (4, W.SR, 8), (1, W.RTN, 16)]


@pytest.mark.parametrize("wid,rounding,window", WINDOW_RUNS)
def test_window_every_head(wid, rounding, window):
    """Pure-write window: the low-bit state, the window's FP8 pairs and scales
    bit-exact at every step, the readout and the exported full state."""
    _run(W.WORKLOADS[wid].scaled(B=2, window=window), 2 * window + 3, rounding=rounding)


def test_window_heads_split_over_waves():
    """B=1: every head is split over several waves, which all read the window
    while the first writes the next copy."""
    w = W.WORKLOADS[0].scaled(window=8, dv=128, steps=20)
    r = _run(w, 20)
    assert r.steps == 20


WINDOW_RAGGED = [
    (W.GDN, W.SR, 64, 37, 16, [8, 4, 4], 8),
    (W.KDA, W.RTN, 256, 45, 32, [4, 8], 4),
    (W.GLA, W.BDR, 128, 70, 64, [8, 4], 16),
    (W.SCALAR, W.SR, 256, 129, 128, [4], 8),
    (W.KDA, W.BDR, 128, 70, 32, [4, 8], 8),
    (W.GDN, W.BDR, 64, 40, 16, [4, 8, 4], 4),
]


@pytest.mark.parametrize("mixer,rounding,dk,dv,G,bits,window", WINDOW_RAGGED)
def test_window_shapes(mixer, rounding, dk, dv, G, bits, window):
    w = W.Workload(65 + mixer, f"win_m{mixer}_dk{dk}_dv{dv}_g{G}_w{window}", mixer, 3, len(bits),
                   dk, dv, G, 2 * window + 2, 3, rounding, "int8", window=window)
    _run(w, 2 * window + 2, hb=np.array(bits, np.uint8), seed=17)


def test_window_full_size_sampled_heads():
    w = W.WORKLOADS[2].scaled(window=8)
    rng = np.random.default_rng(41)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    _run(w, 10, heads=sorted((i // w.H, i % w.H) for i in idx))


BYPASS_RUNS = [(2, W.SR, 8, 0.5), (3, W.RTN, 4, 0.5), (5, W.BDR, 16, 0.5), (4, W.SR, 8, 0.0),
               (1, W.RTN, 4, 2.0), (3, W.SR, 16, 0.25)]


@pytest.mark.parametrize("wid,rounding,window,theta", BYPASS_RUNS)
def test_bypass_every_head(wid, rounding, window, theta):
    """Low-rank bypass: state, buffer pairs and scales bit-exact at every step
    across two merges, the readout and the exported full state."""
    w = W.WORKLOADS[wid].scaled(B=2, window=window, window_merge=1, lrb_threshold=theta)
    _run(w, 2 * window + 3, rounding=rounding)


def test_bypass_heads_split_over_waves():
    w = W.WORKLOADS[0].scaled(window=8, window_merge=1, dv=128, steps=20)
    r = _run(w, 20)
    assert r.steps == 20


@pytest.mark.parametrize("mixer,rounding,dk,dv,G,bits,window", WINDOW_RAGGED)
def test_bypass_shapes(mixer, rounding, dk, dv, G, bits, window):
    w = W.Workload(75 + mixer, f"lrb_m{mixer}_dk{dk}_dv{dv}_g{G}_w{window}", mixer, 3, len(bits),
                   dk, dv, G, 2 * window + 2, 3, rounding, "int8", window=window,
                   window_merge=1, lrb_threshold=0.5)
    _run(w, 2 * window + 2, hb=np.array(bits, np.uint8), seed=19)


def test_bypass_full_size_sampled_heads():
    w = W.WORKLOADS[2].scaled(window=8, window_merge=1)
    rng = np.random.default_rng(43)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    _run(w, 10, heads=sorted((i // w.H, i % w.H) for i in idx))


@pytest.mark.parametrize("layer", [0, 5])
def test_config4_scalar_decay_layers(layer):
    _run(W.WORKLOADS[4].scaled(B=3), 8, layer=layer)


# ragged and edge shapes: dv not a multiple of the rows per iteration, all dk,
# all group sizes, mixed bits in any order, every recurrence and rounding
RAGGED = [
    (W.GDN, W.SR, 64, 37, 16, [8, 4, 4, 8, 4]),
    (W.GDN, W.RTN, 256, 21, 128, [4, 8, 4]),
    (W.GLA, W.SR, 128, 45, 32, [4, 4, 8]),
    (W.SCALAR, W.RTN, 128, 1, 64, [8, 4]),
    (W.SCALAR, W.SR, 256, 70, 16, [4, 8]),
    (W.GDN, W.SR, 128, 129, 128, [4]),
    (W.KDA, W.SR, 64, 53, 32, [8, 4]),
    (W.KDA, W.RTN, 256, 19, 64, [4, 8, 8]),
    (W.GDN, W.BDR, 64, 37, 16, [4, 8, 4]),
    (W.GLA, W.BDR, 256, 23, 128, [8, 4]),
]


@pytest.mark.parametrize("mixer,rounding,dk,dv,G,bits", RAGGED)
def test_ragged_shapes(mixer, rounding, dk, dv, G, bits):
    w = W.Workload(90 + mixer, f"ragged_m{mixer}_dk{dk}_dv{dv}_g{G}", mixer, 3, len(bits), dk, dv,
                   G, 6, 4, rounding, "int8")
    _run(w, 6, hb=np.array(bits, np.uint8), seed=7)


@pytest.mark.parametrize("mixer", [W.GDN, W.GLA, W.SCALAR, W.KDA])
def test_fp32_state_is_the_fp32_recurrence(mixer):
    """The unquantized run equals the reference FP32 recurrence bit for bit."""
    w = W.Workload(95, f"fp32_m{mixer}", mixer, 4, 8, 128, 128, 32, 0, 48, W.RTN, "int8")
    r = Run(w, fp32_only=True)
    log(f"[case] fp32 mixer={mixer} warmup={w.warmup}")
    r.warmup_and_import()


FULL = {1: 3, 2: 2, 3: 2, 4: 2, 5: 2}  # per-channel widths (6): its own test


@pytest.mark.parametrize("wid", sorted(FULL))
def test_full_size_sampled_heads(wid):
    """Full-size launch (the benchmark's shapes); a seeded sample of heads is
    checked against the reference at every step."""
    w = W.WORKLOADS[wid]
    rng = np.random.default_rng(wid)
    idx = set(rng.choice(w.B * w.H, 10, replace=False).tolist()) | {0, w.B * w.H - 1}
    heads = sorted((i // w.H, i % w.H) for i in idx)
    _run(w, FULL[wid], heads=heads)


@pytest.mark.parametrize("window", [0, 8])
def test_bdr_tiny_and_ordinary_groups(window):
    """INT4 bounded directional rounding takes the clamp to [-r, r] only in
    waves holding a group below 2^-100: heads near 1e-35 beside ordinary
    heads (persistent step, and the window step of Gated DeltaNet), every
    head at every step bit-exact."""
    class TinyRun(Run):
        """v scaled by 1e-35 for the heads with even b + h: their states and
        group maxima stay far below 2^-100."""

        def inputs(self, t):
            q, k, v, alpha, beta = super().inputs(t)
            v = v.copy()
            for b in range(self.w.B):
                for h in range(self.w.H):
                    if (b + h) % 2 == 0:
                        v[b, h] *= np.float32(1e-35)
            return q, k, v, alpha, beta

    w = W.Workload(98, "bdr_tiny", W.GDN, 2, 4, 128, 64, 32, 6, 8, W.BDR, "int8").scaled(
        window=window)
    r = TinyRun(w, head_bits_override=np.array([4, 4, 4, 8], np.uint8), seed=3)
    log(f"[case] bdr tiny and ordinary groups window={window}")
    r.warmup_and_import()
    for _ in range(w.steps):
        r.step()
    r.dequant_check()
    r.close()
    assert r.rep.steps == w.steps


def _small_case(mixer=W.GDN, rounding=W.SR, bits=(4, 8, 8)):
    return W.Workload(97, "small", mixer, 2, len(bits), 128, 48, 32, 6, 3, rounding, "int8"), \
        np.array(bits, np.uint8)


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_resume_is_bit_exact():
    """The quantized state is the checkpoint: codes + scales + step counter."""
    w, hb = _small_case()
    cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, w.rounding, False, hb.tolist(), 3, 1)
    rng = np.random.default_rng(3)
    S0 = torch.from_numpy(rng.standard_normal(w.B * w.H * w.dv * w.dk).astype(np.float32)).cuda()
    a = Q.QState(cfg)
    a.load_fp32(S0)
    steps = [W.step_inputs(w, t) for t in range(6)]
    for t in range(3):
        a.step(*map(_dev, steps[t]))
    codes, scales, counter = a.codes.clone(), a.scales.clone(), a.step_counter
    outs_a = []
    for t in range(3, 6):
        o = torch.empty(w.B * w.H * w.dv, device="cuda")
        a.step(*map(_dev, steps[t]), o)
        outs_a.append(o.cpu())
    b = Q.QState(cfg)
    b.codes.copy_(codes)
    b.scales.copy_(scales)
    b.step_counter = counter
    for t in range(3, 6):
        o = torch.empty(w.B * w.H * w.dv, device="cuda")
        b.step(*map(_dev, steps[t]), o)
        assert torch.equal(o.cpu(), outs_a[t - 3])
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert a.step_counter == b.step_counter == 7


def test_guard_bytes_untouched():
    """In-place updates stay inside the caller's buffers."""
    w, hb = _small_case(bits=(4, 8))
    cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, w.rounding, False, hb.tolist(), 0, 0)
    cb, sb = Q.qstate_state_bytes(cfg)
    pad = 4096
    cbuf = torch.full((cb + 2 * pad,), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((sb // 4 + 2 * pad,), 7.25, dtype=torch.float32, device="cuda")
    obuf = torch.full((w.B * w.H * w.dv + 2 * pad,), 3.5, dtype=torch.float32, device="cuda")
    codes, scales = cbuf[pad:pad + cb], sbuf[pad:pad + sb // 4]
    o = obuf[pad:pad + w.B * w.H * w.dv]
    h = Q.qstate_create(cfg, codes, scales)
    S0 = torch.randn(w.B * w.H * w.dv * w.dk, device="cuda")
    Q.qstate_load_fp32(h, S0, cfg)
    for t in range(4):
        q, k, v, alpha, beta = map(_dev, W.step_inputs(w, t))
        Q.qstate_step(h, cfg, q, k, v, alpha, beta, o)
    Q.qstate_readout(h, cfg, q, o)
    torch.cuda.synchronize()
    Q.qstate_destroy(h)
    assert torch.all(cbuf[:pad] == 0xAB) and torch.all(cbuf[pad + cb:] == 0xAB)
    assert torch.all(sbuf[:pad] == 7.25) and torch.all(sbuf[pad + sb // 4:] == 7.25)
    assert torch.all(obuf[:pad] == 3.5) and torch.all(obuf[-pad:] == 3.5)


def test_nan_in_one_row_stays_in_its_head():
    """Heads are independent: a NaN in one head's v leaves every other head
    bit-identical to a clean run."""
    w, hb = _small_case(mixer=W.GDN, bits=(8, 4, 8))
    cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, w.rounding, False, hb.tolist(), 1, 0)
    S0 = torch.randn(w.B * w.H * w.dv * w.dk, device="cuda", generator=None)
    runs = []
    for poison in (False, True):
        a = Q.QState(cfg)
        a.load_fp32(S0)
        for t in range(3):
            q, k, v, alpha, beta = W.step_inputs(w, t)
            if poison and t == 1:
                v = v.copy()
                v[1, 1, 5] = np.nan
            a.step(*map(_dev, (q, k, v, alpha, beta)))
        torch.cuda.synchronize()
        runs.append((a.codes.cpu().numpy(), a.scales.cpu().numpy().reshape(w.B, w.H, -1)))
    ocfg = oracle.cfg(w.B, w.H, w.dk, w.dv, w.G)
    off = oracle.head_offset(ocfg, 1, 1, hb)
    n = w.dv * w.dk * int(hb[1]) // 8
    keep = np.ones(runs[0][0].size, bool)
    keep[off:off + n] = False
    assert np.array_equal(runs[0][0][keep], runs[1][0][keep])
    sk = np.ones((w.B, w.H), bool)
    sk[1, 1] = False
    assert np.array_equal(runs[0][1][sk], runs[1][1][sk])


def test_zero_state_stays_zero():
    w, hb = _small_case(bits=(4, 8))
    for rounding in (W.RTN, W.SR):
        cfg = Q.Config(w.B, w.H, w.dk, w.dv, w.G, w.mixer, rounding, False, hb.tolist(), 0, 0)
        a = Q.QState(cfg)
        a.load_fp32(torch.zeros(w.B * w.H * w.dv * w.dk, device="cuda"))
        q, k, v, alpha, beta = W.step_inputs(w, 0)
        o = torch.full((w.B * w.H * w.dv,), 1.0, device="cuda")
        a.step(*map(_dev, (q, k, np.zeros_like(v), alpha, beta)), o)
        torch.cuda.synchronize()
        assert torch.all(a.codes == 0) and torch.all(a.scales == 0) and torch.all(o == 0)


# ---- limits and extreme magnitudes -----------------------------------------------

def test_most_heads_mixed_bits():
    """256 heads (the most a state may have) with random widths: the per-head
    offset table and INT8 masks up to the last head."""
    rng = np.random.default_rng(51)
    bits = rng.choice([4, 8], 256).astype(np.uint8)
    w = W.Workload(60, "heads256", W.GDN, 2, 256, 64, 16, 16, 3, 2, W.SR, "int8")
    _run(w, 3, hb=bits, seed=3)


def test_most_rows():
    """dv = 4096 rows (the most a head may have), every row checked."""
    w = W.Workload(61, "rows4096", W.KDA, 1, 2, 128, 4096, 32, 2, 2, W.SR, "int8")
    _run(w, 2, hb=np.array([4, 8], np.uint8), seed=5)


@pytest.mark.parametrize("rounding", [W.RTN, W.SR, W.BDR])
def test_extreme_magnitudes(rounding):
    """Rows from about 1e-38 (subnormal scales, the tiny-group paths) up to
    1e30, kept at their magnitude by pure decay steps (write weight 0):
    codes and scales bit-exact, export exact."""
    B, H, dk, dv, G = 1, 2, 128, 48, 32
    hb = np.array([8, 4], np.uint8)
    rng = np.random.default_rng(71)
    mags = np.array([1e-38, 3e-37, 1e-30, 1e-20, 1e-10, 1.0, 1e10, 1e20, 1e30] * 6)[:dv]
    S0 = (rng.standard_normal((B, H, dv, dk)) * mags[None, None, :, None]).astype(np.float32)
    S0[0, 0, 3, :32] = 0.0  # an all-zero group
    cfg = Q.Config(B, H, dk, dv, G, W.SCALAR, rounding, False, hb.tolist(), 9, 2)
    st = Q.QState(cfg)
    st.load_fp32(torch.from_numpy(S0.reshape(-1)).cuda())
    oc = oracle.cfg(B, H, dk, dv, G, W.SCALAR, rounding, 9, 2)
    ref = {}
    for h in range(H):
        ref[h] = oracle.head_quantize(oc, 0, h, int(hb[h]), S0[0, h], 0)[:2]
    for t in range(1, 4):
        q = rng.standard_normal((B, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, dk)).astype(np.float32)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        alpha = np.float32(rng.uniform(0.5, 1.0, (B, H)))
        dt = np.zeros((B, H), np.float32)  # write weight 0: S' = alpha S
        log(f"[case] extreme magnitudes rounding={rounding} step={t}")
        o = torch.empty(B * H * dv, device="cuda")
        st.step(*map(_dev, (q, k, v, alpha, dt)), o)
        torch.cuda.synchronize()
        codes = st.codes.cpu().numpy()
        scales = st.scales.cpu().numpy().reshape(B, H, -1)
        for h in range(H):
            cr, sr = ref[h]
            orr, _, _ = oracle.head_step(oc, 0, h, int(hb[h]), cr, sr, q[0, h], k[0, h], v[0, h],
                                         np.float32([alpha[0, h]]), float(dt[0, h]), step=t)
            off = oracle.head_offset(oc, 0, h, hb)
            assert np.array_equal(scales[0, h].view(np.uint32), sr.view(np.uint32))
            assert np.array_equal(codes[off:off + cr.size], cr)
            og = o.cpu().numpy().reshape(B, H, dv)[0, h]
            assert np.allclose(og, orr, rtol=1e-4, atol=1e-37)
    S = torch.empty(B * H * dv * dk, device="cuda")
    st.store_fp32(S)
    torch.cuda.synchronize()
    Sg = S.cpu().numpy().reshape(B, H, dv, dk)
    for h in range(H):
        assert np.array_equal(Sg[0, h], oracle.head_dequantize(oc, int(hb[h]), *ref[h]))
    st.close()
