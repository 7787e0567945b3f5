"""Pins of the CPU reference's quantized trajectories against the propositions
on the LoReS blog ("LoReS: State Quantization"):

* Prop. "decaying error" (2/4): |E_t|_F <= sum_tau alpha^(t-tau) |eps_tau|_F for
  the delta rule with unit keys, 0 < beta < 2, |alpha|_inf <= alpha < 1;
* Prop. "repeated quantization" (3/4): with scalar decay E_t = sum gamma eps_tau;
  under stochastic rounding the cross terms vanish in expectation, under RTN
  they can reinforce;
* Prop. "per-channel readout error" (1/4): E[e_i^2] = M_i^2 / (12 r^2) under
  value-axis grouping.
"""

import numpy as np
import pytest

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR = 0, 1


def _unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _update64(mixer, X, k, v, alpha, beta):
    X = X.astype(np.float64)
    k64, v64 = k.astype(np.float64), v.astype(np.float64)
    if mixer == GDN:
        return float(alpha) * X @ (np.eye(len(k)) - float(beta) * np.outer(k64, k64)) + \
            float(beta) * np.outer(v64, k64)
    return float(alpha) * X + float(beta) * np.outer(v64, k64)


@pytest.mark.parametrize("bits,rounding", [(4, RTN), (4, SR), (8, SR)])
def test_decaying_error_bound(oracle, bits, rounding):
    rng = np.random.default_rng(60 + bits + rounding)
    dk = dv = 32
    G = 16
    c = oracle.cfg(1, 1, dk, dv, G, mixer=GDN, rounding=rounding, seed=3)
    S0 = (rng.standard_normal((dv, dk)) * 0.5).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S0, step=0)
    Shat = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
    S = S0.astype(np.float64)
    amax = 0.95
    eps_terms = [np.linalg.norm(Shat - S)]  # E_0 = initial quantization error
    for t in range(1, 61):
        k = _unit(rng, dk)
        q = _unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        alpha = np.float32(rng.uniform(0.8, amax))
        beta = float(np.float32(rng.uniform(0.05, 1.95)))
        prev = Shat
        _, pre, _ = oracle.head_step(c, 0, 0, bits, codes, scales, q, k, v,
                                     np.float32([alpha]), beta, step=t, want_pre=True)
        Shat = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        S = _update64(GDN, S, k, v, alpha, beta)
        # the FP32 update of the stored state is the delta rule up to rounding
        eta = np.linalg.norm(pre.astype(np.float64) - _update64(GDN, prev, k, v, alpha, beta))
        assert eta <= 1e-5 * max(1.0, np.linalg.norm(prev))
        eps = np.linalg.norm(Shat - pre.astype(np.float64))
        eps_terms = [amax * e for e in eps_terms] + [eps + eta]
        E = np.linalg.norm(Shat - S)
        assert E <= sum(eps_terms) * (1 + 1e-9) + 1e-12
    # the bound is not vacuous: errors stay at the level of a few fresh errors
    assert np.linalg.norm(Shat - S) < 20 * max(eps_terms)


def _scalar_run(oracle, rounding, seed, coherent, T=100, bits=4):
    """One trajectory S_t = alpha S_{t-1} + dt v_t k_t^T with fixed gates and writes
    (independent of rounding); returns per-step (E_t, eps list, gammas)."""
    dk, dv, G = 32, 8, 32
    c = oracle.cfg(1, 1, dk, dv, G, mixer=SCALAR, rounding=rounding, seed=seed)
    rng = np.random.default_rng(1234)  # same data for every trajectory
    S0 = rng.uniform(-1, 1, (dv, dk)).astype(np.float32)
    S0[:, 0] = 1.0  # keeps each row's absmax, i.e. a nearly fixed grid
    alpha = np.float32(0.995)
    ks = [_unit(rng, dk) for _ in range(T)]
    vs = [rng.standard_normal(dv).astype(np.float32) for _ in range(T)]
    dts = [np.float32(0.002 if coherent else 0.05) for _ in range(T)]
    if coherent:  # the same small write every step: lost by RTN each time
        ks = [ks[0]] * T
        vs = [np.abs(vs[0])] * T
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S0, step=0)
    Shat = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
    S = S0.astype(np.float64)
    eps = [Shat - S]
    R = []
    for t in range(1, T + 1):
        _, pre, _ = oracle.head_step(c, 0, 0, bits, codes, scales, np.zeros(dk, np.float32),
                                     ks[t - 1], vs[t - 1], np.float32([alpha]),
                                     float(dts[t - 1]), step=t, want_pre=True)
        Shat = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        S = _update64(SCALAR, S, ks[t - 1], vs[t - 1], alpha, dts[t - 1])
        eps.append(Shat - pre.astype(np.float64))
        E = Shat - S
        gam = np.array([float(alpha) ** (t - tau) for tau in range(t + 1)])
        # errors propagate linearly: E_t = sum_tau gamma_{tau,t} eps_tau (+ FP32 rounding)
        lin = sum(g * e for g, e in zip(gam, eps))
        assert np.linalg.norm(E - lin) <= 1e-5 * max(1.0, np.linalg.norm(S))
        R.append(np.sum(E**2) - sum(g**2 * np.sum(e**2) for g, e in zip(gam, eps)))
    return np.array(R)


def test_repeated_quantization_cross_terms(oracle):
    # RTN on a coherent write (small updates lost every step): cross terms reinforce.
    r_rtn = _scalar_run(oracle, RTN, 0, coherent=True)
    assert r_rtn[-1] > 0 and np.mean(r_rtn[50:] > 0) > 0.9
    # SR: the same setting, the remainder averages to zero over trajectories.
    runs = np.array([_scalar_run(oracle, SR, s, coherent=True, T=60) for s in range(120)])
    last = runs[:, -1]
    se = last.std(ddof=1) / np.sqrt(len(last))
    assert abs(last.mean()) < 4 * se
    assert abs(last.mean()) < 0.2 * r_rtn[59]


@pytest.mark.parametrize("bits", [4, 8])
def test_readout_error_matches_uniform_model(oracle, bits):
    """Value-axis groups spanning the whole row (G = dk): the readout error of
    RTN has E[e_i^2] = M_i^2 / (12 r^2) for unit q."""
    rng = np.random.default_rng(70 + bits)
    dk = dv = 128
    r = 2 ** (bits - 1) - 1
    c = oracle.cfg(1, 1, dk, dv, dk, rounding=RTN)
    ratios = []
    for head in range(48):
        S = (rng.standard_normal((dv, dk)) * np.exp(rng.uniform(-2, 2, (dv, 1)))).astype(np.float32)
        q = _unit(rng, dk)
        codes, scales, _ = oracle.head_quantize(c, 0, head, bits, S, step=0)
        Shat = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        e = (Shat - S.astype(np.float64)) @ q.astype(np.float64)
        M = np.abs(S).max(axis=1).astype(np.float64)
        ratios.append(e**2 / (M**2 / (12 * r**2)))
    ratio = np.concatenate(ratios).mean()
    assert abs(ratio - 1.0) < 0.05, ratio


def test_batch_wrappers_match_per_head(oracle):
    """The [B][H] entry points slice heads exactly as the per-head ones (mixed bits)."""
    rng = np.random.default_rng(80)
    B, H, dk, dv, G = 2, 3, 64, 16, 32
    hb = np.array([4, 8, 4], np.uint8)
    for mixer in (GDN, GLA, SCALAR):
        c = oracle.cfg(B, H, dk, dv, G, mixer=mixer, rounding=SR, seed=11, layer=4)
        S = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
        codes, scales = oracle.quantize(c, hb, S, 0)
        q = rng.standard_normal((B, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, dk)).astype(np.float32)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        alpha = rng.uniform(0.5, 1, (B, H, dk) if mixer == GLA else (B, H)).astype(np.float32)
        beta = rng.uniform(0, 1, (B, H)).astype(np.float32)
        c2, s2 = codes.copy(), scales.copy()
        o = oracle.step(c, hb, c2, s2, q, k, v, alpha, beta, 1)
        for b in range(B):
            for h in range(H):
                off = oracle.head_offset(c, b, h, hb)
                n = dv * dk * int(hb[h]) // 8
                hc = codes[off:off + n].copy()
                hs = scales[b, h].copy()
                hq, _ = oracle.head_quantize(c, b, h, int(hb[h]), S[b, h], 0)[:2]
                assert np.array_equal(hq, hc)
                a = alpha[b, h] if mixer == GLA else np.float32([alpha[b, h]])
                oh, _, _ = oracle.head_step(c, b, h, int(hb[h]), hc, hs, q[b, h], k[b, h],
                                            v[b, h], a, float(beta[b, h]), step=1)
                assert np.array_equal(hc, c2[off:off + n])
                assert np.array_equal(hs, s2[b, h])
                assert np.array_equal(oh, o[b, h])
        deq = oracle.dequantize(c, hb, c2, s2)
        ro = oracle.readout(c, hb, c2, s2, q)
        for b in range(B):
            for h in range(H):
                assert np.allclose(ro[b, h], deq[b, h].astype(np.float64) @ q[b, h], rtol=1e-5,
                                   atol=1e-5)


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_step_updates_the_stored_state(oracle, mixer, bits):
    """Fig. 1 and "LoReS: State Quantization": the step reads the stored
    (dequantized) state, updates it in full precision and reads out o = S'q
    before requantizing.  Checked against the float64 matrix form."""
    rng = np.random.default_rng(90 + mixer + bits)
    dk, dv, G = 64, 24, 32
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=8)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S0, step=0)
    for t in range(1, 6):
        prev = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        q, k = _unit(rng, dk), _unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        if mixer == GLA:
            alpha = rng.uniform(0.8, 1.0, dk).astype(np.float32)
            beta = 0.0
            want = prev @ np.diag(alpha.astype(np.float64)) + np.outer(v, k).astype(np.float64)
        elif mixer == KDA:
            alpha = rng.uniform(0.8, 1.0, dk).astype(np.float32)
            beta = float(np.float32(rng.uniform(0.1, 1.5)))
            k64 = k.astype(np.float64)
            want = prev @ np.diag(alpha.astype(np.float64)) @ (np.eye(dk) - beta * np.outer(k64, k64)) \
                + beta * np.outer(v.astype(np.float64), k64)
        else:
            alpha = np.float32([rng.uniform(0.8, 1.0)])
            beta = float(np.float32(rng.uniform(0.1, 1.5)))
            want = _update64(mixer, prev, k, v, alpha[0], beta)
        o, pre, _ = oracle.head_step(c, 0, 0, bits, codes, scales, q, k, v, alpha, beta,
                                     step=t, want_pre=True)
        tol = 2e-6 * max(1.0, np.abs(want).max())
        assert np.max(np.abs(pre - want)) <= tol
        assert np.max(np.abs(o - want @ q.astype(np.float64))) <= 8 * tol


@pytest.mark.parametrize("rounding", [RTN, SR])
def test_decaying_error_bound_vector_gates(oracle, rounding):
    """Prop. "decaying error" with vector gates |alpha_t|_inf <= alpha < 1 and
    delta correction (KDA): the accumulated error stays under the geometric
    sum of fresh errors."""
    rng = np.random.default_rng(63 + rounding)
    dk = dv = 32
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=KDA, rounding=rounding, seed=4)
    S0 = (rng.standard_normal((dv, dk)) * 0.5).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, 4, S0, step=0)
    Shat = oracle.head_dequantize(c, 4, codes, scales).astype(np.float64)
    S = S0.astype(np.float64)
    amax = 0.95
    terms = [np.linalg.norm(Shat - S)]
    for t in range(1, 41):
        k, q = _unit(rng, dk), _unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        al = rng.uniform(0.6, amax, dk).astype(np.float32)
        beta = float(np.float32(rng.uniform(0.05, 1.95)))
        k64 = k.astype(np.float64)
        M = np.diag(al.astype(np.float64)) @ (np.eye(dk) - beta * np.outer(k64, k64))
        prev = Shat
        _, pre, _ = oracle.head_step(c, 0, 0, 4, codes, scales, q, k, v, al, beta, step=t,
                                     want_pre=True)
        Shat = oracle.head_dequantize(c, 4, codes, scales).astype(np.float64)
        S = S @ M + beta * np.outer(v.astype(np.float64), k64)
        eta = np.linalg.norm(pre.astype(np.float64) - (prev @ M + beta * np.outer(v, k64)))
        assert eta <= 1e-5 * max(1.0, np.linalg.norm(prev))
        terms = [amax * e for e in terms] + [np.linalg.norm(Shat - pre.astype(np.float64)) + eta]
        assert np.linalg.norm(Shat - S) <= sum(terms) * (1 + 1e-9) + 1e-12
