"""Pins for the full-precision update and readout of the CPU reference.

Update forms: Gated DeltaNet S' = a S (I - b k k^T) + b v k^T (delta rule with
unit keys, 0 < b < 2: LoReS blog, Prop. "decaying error"); GLA
S' = S diag(alpha) + v k^T (vector gates, same proposition's |alpha_t|_inf);
scalar decay S' = a S + dt v k^T (Prop. "repeated quantization", animation
details).  Readout o = S' q (Fig. 1; Prop. "per-channel readout error")."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_2x2_worked.txt")


def _load_golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums], dtype=np.float32)
    return vals


def test_gdn_2x2_worked_example(oracle):
    g = _load_golden()
    c = oracle.cfg(1, 1, 2, 2, 2, mixer=GDN)
    S = g["S"].copy()
    oracle.head_step_fp32(c, S, np.array([0, 1], np.float32), g["k"], g["v"], g["alpha"],
                          float(g["beta"][0]))
    assert np.array_equal(S, g["Snew"])
    # readout of the updated state with q = e1 and q = e0, via a beta = 0,
    # alpha = 1 step (S' = S, exact)
    for qname, q in (("q_e1_o", [0, 1]), ("q_e0_o", [1, 0])):
        S2 = g["Snew"].copy()
        o = oracle.head_step_fp32(c, S2, np.array(q, np.float32), g["k"], g["v"],
                                  np.float32([1.0]), 0.0)
        assert np.array_equal(o, g[qname])
        assert np.array_equal(S2, g["Snew"])


def _rand_unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _fp64_step(mixer, S, q, k, v, alpha, beta):
    """Matrix form of the update, float64."""
    S = S.astype(np.float64)
    k64, q64, v64 = k.astype(np.float64), q.astype(np.float64), v.astype(np.float64)
    if mixer == GDN:
        a, b = float(alpha[0]), float(beta)
        Sn = a * S @ (np.eye(len(k)) - b * np.outer(k64, k64)) + b * np.outer(v64, k64)
    elif mixer == GLA:
        Sn = S @ np.diag(alpha.astype(np.float64)) + np.outer(v64, k64)
    elif mixer == KDA:
        b = float(beta)
        Sn = S @ np.diag(alpha.astype(np.float64)) @ (np.eye(len(k)) - b * np.outer(k64, k64)) \
            + b * np.outer(v64, k64)
    else:
        Sn = float(alpha[0]) * S + float(beta) * np.outer(v64, k64)
    return Sn, Sn @ q64


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 48), (128, 128)])
def test_fp32_recurrence_tracks_float64_matrix_form(oracle, mixer, dk, dv):
    rng = np.random.default_rng(10 + mixer)
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=mixer)
    S = (rng.standard_normal((dv, dk)) * 0.3).astype(np.float32)
    S64 = S.astype(np.float64)
    for t in range(40):
        q, k = _rand_unit(rng, dk), _rand_unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        if mixer in (GLA, KDA):
            alpha = (1 / (1 + np.exp(-(rng.standard_normal(dk) + 3)))) ** (1 / 16)
            alpha = alpha.astype(np.float32)
            beta = 0.0 if mixer == GLA else float(np.float32(1 / (1 + math.exp(-rng.standard_normal()))))
        else:
            alpha = np.float32([math.exp(-math.log1p(math.exp(rng.standard_normal() - 4)))])
            beta = float(np.float32(1 / (1 + math.exp(-rng.standard_normal()))))
        o = oracle.head_step_fp32(c, S, q, k, v, alpha, beta)
        S64, o64 = _fp64_step(mixer, S64, q, k, v, alpha, beta)
        scale = np.abs(S64).max()
        assert np.max(np.abs(S - S64)) <= 2e-5 * max(scale, 1.0)
        assert np.max(np.abs(o - o64)) <= 2e-5 * max(np.abs(o64).max(), 1.0)


def test_gdn_closed_forms(oracle):
    """(i) S'k = a(1-b)Sk + b v for unit k; (ii) S'x = a S x for x orthogonal to k;
    (iii) b = 0 gives S' = a S; a = 1, b = 0 is the identity."""
    rng = np.random.default_rng(20)
    dk = dv = 32
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=GDN)
    for _ in range(10):
        S0 = rng.standard_normal((dv, dk)).astype(np.float32)
        k = _rand_unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        a = np.float32(rng.uniform(0.8, 1.0))
        b = float(np.float32(rng.uniform(0.1, 1.9)))
        S = S0.copy()
        oracle.head_step_fp32(c, S, k, k, v, np.float32([a]), b)
        S0d, Sd, kd = S0.astype(np.float64), S.astype(np.float64), k.astype(np.float64)
        lhs = Sd @ kd
        rhs = float(a) * (1 - b) * (S0d @ kd) + b * v
        assert np.allclose(lhs, rhs, rtol=0, atol=2e-5 * np.abs(S0).max() * 4)
        x = rng.standard_normal(dk)
        x -= (x @ kd) * kd
        assert np.allclose(Sd @ x, float(a) * (S0d @ x), atol=2e-5 * np.abs(S0).max() * 6)
        # beta = 1 writes v exactly along k (up to rounding)
        S = S0.copy()
        oracle.head_step_fp32(c, S, k, k, v, np.float32([a]), 1.0)
        assert np.allclose(S.astype(np.float64) @ kd, v, atol=1e-4 * max(1, np.abs(S0).max()))
    S = S0.copy()
    oracle.head_step_fp32(c, S, k, k, v, np.float32([0.75]), 0.0)
    assert np.array_equal(S, (S0 * np.float32(0.75)) + np.float32(0))
    S = S0.copy()
    oracle.head_step_fp32(c, S, k, k, v, np.float32([1.0]), 0.0)
    assert np.array_equal(S, S0)


def test_gdn_orthonormal_keys_closed_form(oracle):
    """4x4, keys e0..e3 in turn, beta = 1, S0 = 0:
    S_T = sum_t (prod_{tau > t} alpha_tau) v_t e_t^T."""
    c = oracle.cfg(1, 1, 4, 4, 4, mixer=GDN)
    rng = np.random.default_rng(30)
    S = np.zeros((4, 4), np.float32)
    alphas = [0.5, 0.75, 0.25, 0.875]
    vs = [rng.integers(-8, 8, 4).astype(np.float32) for _ in range(4)]
    for t in range(4):
        e = np.zeros(4, np.float32)
        e[t] = 1
        oracle.head_step_fp32(c, S, e, e, vs[t], np.float32([alphas[t]]), 1.0)
    expect = np.zeros((4, 4), np.float64)
    for t in range(4):
        expect[:, t] = np.prod(alphas[t + 1:]) * vs[t]
    assert np.array_equal(S.astype(np.float64), expect)  # dyadic: exact


def test_gla_closed_form(oracle):
    """S_T = sum_t v_t (k_t o prod_{tau>t} alpha_tau)^T from S0 = 0 (exact, dyadic)."""
    dk, dv = 16, 8
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=GLA)
    rng = np.random.default_rng(31)
    S = np.zeros((dv, dk), np.float32)
    ks, vs, als = [], [], []
    for t in range(5):
        k = rng.integers(-4, 5, dk).astype(np.float32)
        v = rng.integers(-4, 5, dv).astype(np.float32)
        al = rng.choice([0.5, 0.75, 1.0, 0.875], dk).astype(np.float32)
        oracle.head_step_fp32(c, S, np.zeros(dk, np.float32), k, v, al, 0.0)
        ks.append(k), vs.append(v), als.append(al)
    expect = np.zeros((dv, dk))
    for t in range(5):
        decay = np.prod(np.array(als[t + 1:], dtype=np.float64), axis=0) if t < 4 else 1.0
        expect += np.outer(vs[t], ks[t] * decay)
    assert np.array_equal(S.astype(np.float64), expect)


def test_scalar_decay_closed_form(oracle):
    """S_T = sum_t gamma_{t,T} dt_t v_t k_t^T with gamma_{t,T} = prod_{tau>t} alpha_tau
    (Prop. "repeated quantization"), exact on dyadic data."""
    dk, dv = 16, 4
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=SCALAR)
    rng = np.random.default_rng(32)
    S = np.zeros((dv, dk), np.float32)
    terms = []
    alphas = [0.5, 0.75, 0.875, 0.5, 0.25]
    for t in range(5):
        k = rng.integers(-4, 5, dk).astype(np.float32)
        v = rng.integers(-4, 5, dv).astype(np.float32)
        dt = [0.5, 0.25, 1.0, 0.125, 0.5][t]
        oracle.head_step_fp32(c, S, np.zeros(dk, np.float32), k, v, np.float32([alphas[t]]), dt)
        terms.append((dt, v, k))
    expect = np.zeros((dv, dk))
    for t, (dt, v, k) in enumerate(terms):
        expect += np.prod(alphas[t + 1:]) * dt * np.outer(v, k)
    assert np.array_equal(S.astype(np.float64), expect)


def test_single_error_survival_alpha_pow_n(oracle):
    """LoReS 2/4 animation: one injected error, constant scalar decay, no further
    rounding: |E_n|_F / |E_0|_F = alpha^n (exact on dyadic data, alpha = 1/2)."""
    dk, dv = 16, 16
    c = oracle.cfg(1, 1, dk, dv, 16, mixer=SCALAR)
    rng = np.random.default_rng(33)
    S = rng.integers(-64, 64, (dv, dk)).astype(np.float32)
    E0 = rng.integers(-64, 64, (dv, dk)).astype(np.float32)
    Sa, Sb = S.copy(), S + E0
    for n in range(1, 9):
        k = rng.integers(-2, 3, dk).astype(np.float32)
        v = rng.integers(-2, 3, dv).astype(np.float32)
        for X in (Sa, Sb):
            oracle.head_step_fp32(c, X, np.zeros(dk, np.float32), k, v, np.float32([0.5]), 0.25)
        ratio = np.linalg.norm((Sb - Sa).astype(np.float64)) / np.linalg.norm(E0.astype(np.float64))
        assert ratio == 0.5**n
    # and approximately for a generic alpha
    a = 0.93
    Sa, Sb = S.copy(), S + E0 * 1e-3
    for n in range(1, 30):
        k = _rand_unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        for X in (Sa, Sb):
            oracle.head_step_fp32(c, X, np.zeros(dk, np.float32), k, v, np.float32([a]), 0.1)
    ratio = np.linalg.norm((Sb - Sa).astype(np.float64)) / np.linalg.norm(E0 * 1e-3)
    assert abs(ratio / float(np.float32(a)) ** 29 - 1) < 2e-3


def test_dot_error_bound_and_exact_cases(oracle):
    rng = np.random.default_rng(40)
    u = 2.0**-24
    for n in (1, 5, 16, 17, 64, 100, 128, 256):
        for _ in range(20):
            x = rng.standard_normal(n).astype(np.float32)
            y = rng.standard_normal(n).astype(np.float32)
            got = Fraction(float(oracle.dot(x, y)))
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, y))
            depth = min(n, 16) + math.ceil(math.log2(max(1, math.ceil(n / 16)))) + 1
            gamma = depth * u / (1 - depth * u)
            bound = Fraction(gamma) * sum(abs(Fraction(float(a)) * Fraction(float(b)))
                                          for a, b in zip(x, y))
            assert abs(got - exact) <= bound
        # small integers: exact in any order
        xi = rng.integers(-100, 100, n).astype(np.float32)
        yi = rng.integers(-100, 100, n).astype(np.float32)
        assert oracle.dot(xi, yi) == float(np.dot(xi.astype(np.int64), yi.astype(np.int64)))
        # unit vectors select one entry exactly
        j = int(rng.integers(0, n))
        e = np.zeros(n, np.float32)
        e[j] = 1
        assert oracle.dot(x, e) == x[j]


def test_kda_reduces_to_delta_rule_and_to_gla(oracle):
    """KDA (per-channel decay + delta correction; LoReS Table 1 "KDA") with a
    uniform gate is the Gated DeltaNet step, and with beta = 0 it is the GLA
    decay alone (GLA's step with v = 0): bit-identical in FP32 and quantized."""
    rng = np.random.default_rng(41)
    dk, dv = 64, 32
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    q, k = _rand_unit(rng, dk), _rand_unit(rng, dk)
    v = rng.standard_normal(dv).astype(np.float32)
    a = np.float32(0.9375)
    b = float(np.float32(0.625))
    ck, cg = oracle.cfg(1, 1, dk, dv, 32, mixer=KDA), oracle.cfg(1, 1, dk, dv, 32, mixer=GDN)
    X, Y = S0.copy(), S0.copy()
    ox = oracle.head_step_fp32(ck, X, q, k, v, np.full(dk, a, np.float32), b)
    oy = oracle.head_step_fp32(cg, Y, q, k, v, np.float32([a]), b)
    # c*(s*a) and (c*s)*a differ in rounding, so compare the FP32 form (S*a both ways)
    assert np.array_equal(X, Y) and np.array_equal(ox, oy)
    al = rng.uniform(0.8, 1.0, dk).astype(np.float32)
    cl = oracle.cfg(1, 1, dk, dv, 32, mixer=GLA)
    X, Y = S0.copy(), S0.copy()
    oracle.head_step_fp32(ck, X, q, k, v, al, 0.0)
    oracle.head_step_fp32(cl, Y, q, k, np.zeros(dv, np.float32), al, 0.0)
    assert np.array_equal(X, Y)
    for bits in (4, 8):
        codes, scales, _ = oracle.head_quantize(ck, 0, 0, bits, S0, 0)
        c1, s1, c2, s2 = codes.copy(), scales.copy(), codes.copy(), scales.copy()
        o1, _, _ = oracle.head_step(ck, 0, 0, bits, c1, s1, q, k, v, al, 0.0, step=1)
        o2, _, _ = oracle.head_step(cl, 0, 0, bits, c2, s2, q, k, np.zeros(dv, np.float32), al,
                                    0.0, step=1)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(o1, o2)
