"""Pins for the pure-write window in the CPU reference.

"Low-Bit GDN Recurrent-State Quantization: Global Gradient-aware Allocation
and Pure-Write Sliding Windows" (abstract): the last W pure writes are kept
as FP8 vector pairs beside the low-bit state, propagated through the full
state transition, and merged into the low-bit state only after they leave
the window.  Pinned here: the OCP E4M3 format (decode table from the format
definition, encoding by brute force), that a window holding every write of
a trajectory reproduces the plain FP32 recurrence up to FP8 error, that an
empty window is the plain quantized step, that a merged pair lands in the
state it leaves for, and that the window lowers the readout error of a
low-bit state."""

from fractions import Fraction

import numpy as np
import pytest

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2


def _e4m3(code):
    """OCP E4M3 from its definition (exact rational), None for NaN."""
    s = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2**6)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def test_fp8_decode_is_e4m3(oracle):
    finite = 0
    for code in range(256):
        want = _e4m3(code)
        got = oracle.fp8_decode(code)
        if want is None:
            assert np.isnan(got)
        else:
            assert Fraction(float(got)) == want, code
            finite += 1
    assert finite == 254
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(1) == 2.0**-9


def test_fp8_encode_is_nearest_even(oracle):
    grid = sorted({_e4m3(c) for c in range(0x7F)})
    rng = np.random.default_rng(500)
    xs = [float(np.float32(x)) for x in rng.uniform(-448, 448, 2000)]
    xs += [float(np.float32(x)) for x in np.exp(rng.uniform(np.log(1e-4), np.log(448), 3000))]
    # every midpoint between neighbours (exact ties) and its float neighbours
    for a, b in zip(grid[:-1], grid[1:]):
        mid = float((a + b) / 2)
        xs += [mid, float(np.nextafter(np.float32(mid), np.float32(0))),
               float(np.nextafter(np.float32(mid), np.float32(1000)))]
    xs += [0.0, 448.0, 2.0**-10, 2.0**-12]
    for x in xs:
        for sx in (x, -x):
            code = oracle.fp8_encode(sx)
            ax = abs(Fraction(sx))
            errs = [(abs(g - ax), g) for g in grid]
            best = min(e for e, _ in errs)
            cands = [c for c in range(0x7F) if abs(_e4m3(c) - ax) == best]
            pick = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
            assert code & 0x7F == pick, (sx, code, cands)
            assert (code >> 7) == (1 if np.signbit(np.float32(sx)) else 0)


def _unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _inputs(rng, mixer, dk, dv):
    q, k = _unit(rng, dk), _unit(rng, dk)
    v = rng.standard_normal(dv).astype(np.float32)
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


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
def test_window_holding_every_write_is_the_recurrence(oracle, mixer):
    """From a zero state with W >= T steps nothing is merged: H stays zero and
    the pairs alone carry the state, which then equals the float64
    recurrence up to the FP8 rounding of the pairs; the readouts likewise."""
    rng = np.random.default_rng(520 + mixer)
    dk, dv, G, W, T = 64, 32, 32, 8, 8
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=1, window=W)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, 4, np.zeros((dv, dk), np.float32), 0)
    win = np.zeros(oracle.window_bytes(c), np.uint8)
    S = np.zeros((dv, dk))
    for t in range(1, T + 1):
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        o, pre, _ = oracle.head_step_pw(c, 0, 0, 4, codes, scales, win, q, k, v, alpha, beta,
                                        step=t, want_pre=True)
        S = _update64(mixer, S, q, k, v, alpha, beta)
        assert np.all(pre == 0)  # nothing merged yet: H stays zero
        assert np.allclose(o, S @ q.astype(np.float64), atol=0.08 * np.abs(S).max() + 1e-6)
        full = oracle.head_window_state(c, 4, codes, scales, win, t + 1)
        rel = np.linalg.norm(full - S) / np.linalg.norm(S)
        # E4M3 keeps 3 mantissa bits (relative error <= 2^-4 per value, about
        # 3.6 % rms); a pair's key is re-encoded every step it ages, so the
        # error of the oldest pairs grows with sqrt(T): 0.12 at T = 8
        assert rel < 0.12, rel


@pytest.mark.parametrize("rounding", [RTN, SR, BDR])
def test_empty_window_is_the_plain_step(oracle, rounding):
    """With every slot empty (zero scales) the first step equals the plain
    quantized step bit for bit, readout included."""
    rng = np.random.default_rng(540 + rounding)
    dk, dv, G = 64, 24, 16
    for mixer in (GDN, GLA, SCALAR, KDA):
        c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=rounding, seed=4, window=4)
        c0 = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=rounding, seed=4)
        S0 = rng.standard_normal((dv, dk)).astype(np.float32)
        a_codes, a_scales, _ = oracle.head_quantize(c, 0, 0, 8, S0, 0)
        b_codes, b_scales = a_codes.copy(), a_scales.copy()
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        win = np.zeros(oracle.window_bytes(c), np.uint8)
        o1, p1, _ = oracle.head_step_pw(c, 0, 0, 8, a_codes, a_scales, win, q, k, v, alpha, beta,
                                        step=1, want_pre=True)
        o0, p0, _ = oracle.head_step(c0, 0, 0, 8, b_codes, b_scales, q, k, v, alpha, beta,
                                     step=1, want_pre=True)
        # H' differs from the plain S' by exactly the pure write, now in the window
        wv = (v if mixer == GLA else np.float32(beta) * v).astype(np.float64)
        assert np.max(np.abs(p1 + np.outer(wv, k) - p0)) < 1e-5 * max(1.0, np.abs(p0).max())
        assert np.allclose(o1, o0, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("mixer", [GDN, KDA])
def test_leaving_pair_is_merged(oracle, mixer):
    """The step's pre-quantization state is H A + a_o b_o'^T with the pair in
    slot `step mod W` (oldest), checked in float64 from the stored window."""
    rng = np.random.default_rng(560 + mixer)
    dk, dv, G, W = 64, 32, 32, 4
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=2, window=W)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, 8, rng.standard_normal((dv, dk)).astype(np.float32), 0)
    win = np.zeros(oracle.window_bytes(c), np.uint8)
    for t in range(1, 11):
        q, k, v, alpha, beta = _inputs(rng, mixer, dk, dv)
        H = oracle.head_dequantize(c, 8, codes, scales).astype(np.float64)
        full = oracle.head_window_state(c, 8, codes, scales, win, t).astype(np.float64)

        # decode the oldest pair directly from the bytes
        slot = t % W
        a8 = win[:dv * W].reshape(dv, W)[:, slot]
        b8 = win[dv * W:dv * W + W * dk].reshape(W, dk)[slot]
        sc = win[dv * W + W * dk:dv * W + W * dk + 8 * W].view(np.float32).reshape(W, 2)[slot]
        a = np.array([oracle.fp8_decode(int(x)) for x in a8]) * sc[0]
        b = np.array([oracle.fp8_decode(int(x)) for x in b8]) * sc[1]
        o, pre, _ = oracle.head_step_pw(c, 0, 0, 8, codes, scales, win, q, k, v, alpha, beta,
                                        step=t, want_pre=True)
        k64 = k.astype(np.float64)
        Dh = H * alpha.astype(np.float64)[None, :] if alpha.size > 1 else H * float(alpha[0])
        Ah = Dh - beta * np.outer(Dh @ k64, k64)
        db = b * (alpha.astype(np.float64) if alpha.size > 1 else float(alpha[0]))
        bp = db - beta * k64 * (db @ k64)
        want = Ah + np.outer(a, bp)
        assert np.max(np.abs(pre - want)) < 2e-5 * max(1.0, np.abs(want).max())
        # readout of the full state: H' q plus the pairs still in the window
        Sfull = _update64(mixer, full, q, k, v, alpha, beta)
        assert np.allclose(o, Sfull @ q.astype(np.float64), atol=1e-3 * np.abs(Sfull).max())


def test_window_lowers_readout_error(oracle):
    """The point of the window: recent writes kept at FP8 beside an INT4
    state give readouts closer to the FP32 recurrence than the INT4 state
    alone (same trajectory, same rounding)."""
    dk, dv, G, T = 64, 32, 32, 64
    err = {}
    for W in (0, 8):
        e = 0.0
        for rep in range(4):
            rng = np.random.default_rng(600 + rep)
            c = oracle.cfg(1, 1, dk, dv, G, mixer=GDN, rounding=SR, seed=rep, window=W)
            codes, scales, _ = oracle.head_quantize(c, 0, 0, 4, np.zeros((dv, dk), np.float32), 0)
            win = np.zeros(oracle.window_bytes(c) if W else 16, np.uint8)
            S = np.zeros((dv, dk))
            for t in range(1, T + 1):
                q, k, v, alpha, beta = _inputs(rng, GDN, dk, dv)
                alpha = np.float32([0.98])
                if W:
                    o, _, _ = oracle.head_step_pw(c, 0, 0, 4, codes, scales, win, q, k, v, alpha,
                                                  beta, step=t)
                else:
                    o, _, _ = oracle.head_step(c, 0, 0, 4, codes, scales, q, k, v, alpha, beta,
                                               step=t)
                S = _update64(GDN, S, q, k, v, alpha, beta)
                if t > T // 2:
                    e += float(np.sum((o - S @ q.astype(np.float64)) ** 2))
        err[W] = e
    assert err[8] < 0.8 * err[0], err
