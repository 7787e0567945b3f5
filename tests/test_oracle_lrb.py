"""Pins for the low-rank bypass in the CPU reference.

"Preserving Updates in Low-Bit Recurrent State Quantization" (abstract):
small updates accumulate in a compact low-rank buffer, whose sufficiently
large elements are merged into the state periodically.  Read here as the
pair buffer of the pure-write window (the W most recent writes, propagated
through the transition) merged as a whole every W steps, elements below a
threshold times their group scale dropped.  Pinned: one slot with threshold
0 is the window of one pair; an infinite threshold is the plain step
without its write; threshold 0 keeps the float64 recurrence; the threshold
picks elements by their magnitude against the stored scale; merges happen
exactly at counters that are multiples of W and leave only the new pair;
a step between merges is the window step."""

import numpy as np
import pytest

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2


def _unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _inputs(rng, mixer, dk, dv, vscale=1.0):
    q, k = _unit(rng, dk), _unit(rng, dk)
    v = (vscale * rng.standard_normal(dv)).astype(np.float32)
    if mixer in (GLA, KDA):
        alpha = rng.uniform(0.85, 1.0, dk).astype(np.float32)
    else:
        alpha = np.float32([rng.uniform(0.85, 1.0)])
    beta = 0.0 if mixer == GLA else float(np.float32(rng.uniform(0.2, 1.2)))
    return q, k, v, alpha, beta


def _update64(mixer, S, q, k, v, alpha, beta):
    k64, v64 = k.astype(np.float64), v.astype(np.float64)
    D = S * alpha.astype(np.float64)[None, :] if alpha.size > 1 else S * float(alpha[0])
    if mixer in (GDN, KDA):
        return D - beta * np.outer(D @ k64, k64) + beta * np.outer(v64, k64)
    w = 1.0 if mixer == GLA else beta
    return D + w * np.outer(v64, k64)


def _slot_scales(c, win):
    W, dv, dk = c.window, c.dv, c.dk
    off = dv * W + W * dk
    return win[off:off + 8 * W].view(np.float32).reshape(W, 2)


def _filled(oracle, c, bits, rng, mixer, steps, seed_state=True):
    """A head after an import at counter 0 and `steps` bypass steps."""
    S0 = rng.standard_normal((c.dv, c.dk)).astype(np.float32) if seed_state else \
        np.zeros((c.dv, c.dk), np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S0, 0)
    win = np.zeros(oracle.window_bytes(c), np.uint8)
    for t in range(1, steps + 1):
        q, k, v, alpha, beta = _inputs(rng, mixer, c.dk, c.dv)
        oracle.head_step_pw(c, 0, 0, bits, codes, scales, win, q, k, v, alpha, beta, step=t)
    return codes, scales, win


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
def test_one_slot_zero_threshold_is_the_window_of_one(oracle, mixer):
    """W = 1 merges every step; with threshold 0 every element merges, which
    is the window of one pair up to adding the merged term after the
    transition (two roundings) instead of inside it (one)."""
    rng = np.random.default_rng(700 + mixer)
    dk, dv, G = 64, 32, 32
    cl = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=3, window=1,
                    window_merge=1, lrb_threshold=0.0)
    cw = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=3, window=1)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(cl, 0, 0, 8, S0, 0)
    win = np.zeros(oracle.window_bytes(cl), np.uint8)
    for t in range(1, 7):
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        c2, s2, w2 = codes.copy(), scales.copy(), win.copy()
        o1, p1, _ = oracle.head_step_pw(cl, 0, 0, 8, codes, scales, win, q, k, v, alpha, beta,
                                        step=t, want_pre=True)
        o2, p2, _ = oracle.head_step_pw(cw, 0, 0, 8, c2, s2, w2, q, k, v, alpha, beta,
                                        step=t, want_pre=True)
        tol = 4 * np.finfo(np.float32).eps * max(1.0, float(np.abs(p2).max()))
        assert np.max(np.abs(p1 - p2)) <= tol
        assert np.allclose(o1, o2, rtol=1e-5, atol=1e-5)
        # carry the window's result on, so both see the same start next step
        codes, scales, win = c2, s2, w2


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
@pytest.mark.parametrize("rounding", [RTN, SR, BDR])
def test_infinite_threshold_drops_the_buffer(oracle, mixer, rounding):
    """At a merge step with an infinite threshold nothing merges: the state
    is the plain quantized step with a zero write, bit for bit, and the
    buffer keeps only the new pair."""
    rng = np.random.default_rng(720 + 4 * mixer + rounding)
    dk, dv, G, W = 64, 24, 16, 4
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=rounding, seed=5, window=W,
                   window_merge=1, lrb_threshold=np.inf)
    c0 = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=rounding, seed=5)
    codes, scales, win = _filled(oracle, c, 8, rng, mixer, W - 1)
    assert np.count_nonzero(_slot_scales(c, win)) > 0  # the buffer holds pairs
    b_codes, b_scales = codes.copy(), scales.copy()
    q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
    o1, _, _ = oracle.head_step_pw(c, 0, 0, 8, codes, scales, win, q, k, v, alpha, beta, step=W)
    o0, _, _ = oracle.head_step(c0, 0, 0, 8, b_codes, b_scales, q, k, np.zeros_like(v), alpha,
                                beta, step=W)
    assert np.array_equal(codes, b_codes) and np.array_equal(scales, b_scales)
    wv = (v if mixer == GLA else np.float32(beta) * v).astype(np.float64)
    assert np.allclose(o1 - wv * float(k.astype(np.float64) @ q), o0, rtol=1e-5, atol=1e-5)
    sc = _slot_scales(c, win)
    assert np.all(sc[1:] == 0) and sc[0, 1] > 0


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
def test_zero_threshold_keeps_the_recurrence(oracle, mixer):
    """Threshold 0 merges every element, so H + buffer follows the float64
    recurrence across several merges, up to INT8 and FP8 rounding."""
    rng = np.random.default_rng(740 + mixer)
    dk, dv, G, W, T = 64, 32, 32, 4, 13
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=6, window=W,
                   window_merge=1, lrb_threshold=0.0)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, 8, S0, 0)
    S = oracle.head_dequantize(c, 8, codes, scales).astype(np.float64)
    win = np.zeros(oracle.window_bytes(c), np.uint8)
    for t in range(1, T + 1):
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        o, _, _ = oracle.head_step_pw(c, 0, 0, 8, codes, scales, win, q, k, v, alpha, beta, step=t)
        S = _update64(mixer, S, q, k, v, alpha, beta)
        full = oracle.head_window_state(c, 8, codes, scales, win, t + 1)
        rel = np.linalg.norm(full - S) / np.linalg.norm(S)
        # INT8 stochastic rounding adds about 0.8 % (rms, relative) per
        # step and re-encoding the pairs' keys in E4M3 about 0.5 %; they
        # add up as a random walk.  Dropping the buffer at a merge would
        # cost the 4 writes' share of the state, over 10 %.
        assert rel < 0.012 * np.sqrt(t), (t, rel)
        assert np.allclose(o, S @ q.astype(np.float64), atol=0.03 * np.abs(S).max())


@pytest.mark.parametrize("mixer", [GDN, GLA, KDA])
def test_threshold_selects_by_magnitude_against_stored_scale(oracle, mixer):
    """At a merge step each element takes the threshold-0 value when the
    merged term reaches threshold * (its stored group scale before the step)
    and the infinite-threshold value otherwise."""
    rng = np.random.default_rng(760 + mixer)
    dk, dv, G, W = 64, 32, 16, 8
    theta = 0.5
    cfgs = {th: oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=7, window=W,
                           window_merge=1, lrb_threshold=th) for th in (0.0, theta, np.inf)}
    codes, scales, win = _filled(oracle, cfgs[theta], 4, rng, mixer, W - 1)
    s_old = np.repeat(scales.reshape(dv, dk // G), G, axis=1).astype(np.float64)
    q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
    pre = {}
    for th, c in cfgs.items():
        c2, s2, w2 = codes.copy(), scales.copy(), win.copy()
        _, pre[th], _ = oracle.head_step_pw(c, 0, 0, 4, c2, s2, w2, q, k, v, alpha, beta,
                                            step=W, want_pre=True)
    m = pre[0.0].astype(np.float64) - pre[np.inf].astype(np.float64)
    thr = theta * s_old
    clear = np.abs(np.abs(m) - thr) > 1e-4 * (np.abs(m) + thr)
    sel = (np.abs(m) >= thr) & clear
    keep = (np.abs(m) < thr) & clear
    assert sel.sum() > 20 and keep.sum() > 20, (sel.sum(), keep.sum())
    assert np.array_equal(pre[theta][sel], pre[0.0][sel])
    assert np.array_equal(pre[theta][keep], pre[np.inf][keep])


def test_merge_period_and_emptying(oracle):
    """After an import at counter 0 the pair of counter t sits in slot
    t mod W; the step at every multiple of W merges the buffer and leaves
    only its own pair (slot 0)."""
    rng = np.random.default_rng(780)
    dk, dv, G, W = 64, 16, 32, 4
    c = oracle.cfg(1, 1, dk, dv, G, mixer=GDN, rounding=RTN, window=W, window_merge=1)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, 8, rng.standard_normal((dv, dk)).astype(np.float32), 0)
    win = np.zeros(oracle.window_bytes(c), np.uint8)
    for t in range(1, 3 * W + 2):
        q, k, v, alpha, beta = _inputs(rng, GDN, dk, dv)
        oracle.head_step_pw(c, 0, 0, 8, codes, scales, win, q, k, v, alpha, beta, step=t)
        live = set(np.nonzero(_slot_scales(c, win)[:, 1])[0].tolist())
        first = 0 if t >= W else 1
        want = set(range(first, t % W + 1)) if t % W else {0}
        assert live == want, (t, live, want)
        if t % W == 0:  # emptied slots hold zero codes too
            a = win[:dv * W].reshape(dv, W)
            b = win[dv * W:dv * W + W * dk].reshape(W, dk)
            assert np.all(a[:, 1:] == 0) and np.all(b[1:] == 0)


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
def test_step_between_merges_is_the_window_step(oracle, mixer):
    """Away from multiples of W the bypass step is the pure-write window
    step (whose leaving slot is then empty), bit for bit."""
    rng = np.random.default_rng(800 + mixer)
    dk, dv, G, W = 64, 32, 32, 8
    cl = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=9, window=W,
                    window_merge=1)
    cw = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=9, window=W)
    codes, scales, win = _filled(oracle, cl, 4, rng, mixer, W + 2)
    for t in range(W + 3, 2 * W):
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        c2, s2, w2 = codes.copy(), scales.copy(), win.copy()
        o1, _, _ = oracle.head_step_pw(cl, 0, 0, 4, codes, scales, win, q, k, v, alpha, beta, step=t)
        o2, _, _ = oracle.head_step_pw(cw, 0, 0, 4, c2, s2, w2, q, k, v, alpha, beta, step=t)
        assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
        assert np.array_equal(win, w2) and np.array_equal(o1, o2)
