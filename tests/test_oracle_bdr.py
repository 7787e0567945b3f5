"""Pins for bounded directional rounding (BDR) in the CPU reference.

"Preserving Updates in Low-Bit Recurrent State Quantization" (abstract): a
state element can move opposite to its update when it is requantized; BDR
rounds such reversed elements toward their update, needs no storage beyond
the state, and enlarges the rounding error.  The element-level rule is
pinned by hand-derived dyadic cases (tests/golden/bdr_cases.txt); the step
is pinned by what the rule must guarantee on whole trajectories: every code
stays one of the two grid neighbours of the exact scaled value, no stored
value moves against its update, every other element is rounded to nearest,
and the mean rounding error grows."""

from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import workloads as W

GOLDEN = Path(__file__).parent / "golden" / "bdr_cases.txt"


def _cases():
    out = []
    for line in GOLDEN.read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        out.append((float(f[0]), float(f[1]), float(f[2]), float(f[3]), int(f[4]), int(f[5]),
                    int(f[6]), " ".join(f[7:])))
    return out


@pytest.mark.parametrize("prev,x,s_new,inv,r,rtn,bdr,what", _cases())
def test_bdr_golden_cases(oracle, prev, x, s_new, inv, r, rtn, bdr, what):
    assert oracle.round_rtn(x, inv) == rtn, what
    assert oracle.round_bdr(x, inv, s_new, prev, r) == bdr, what


def _unpack(codes, bits, dv, dk):
    if bits == 8:
        return codes.view(np.int8).astype(np.int64).reshape(dv, dk)
    x = np.empty(codes.size * 2, np.int64)
    x[0::2], x[1::2] = codes & 0xF, codes >> 4
    x[x >= 8] -= 16
    return x.reshape(dv, dk)


def _nearest_even(t):
    """Round-half-even of exact rationals (brute force over the two neighbours)."""
    out = np.empty(len(t), np.int64)
    for n, v in enumerate(t):
        fl = v.numerator // v.denominator
        fr = v - fl
        out[n] = fl + 1 if (fr > Fraction(1, 2) or (fr == Fraction(1, 2) and fl % 2)) else fl
    return out


def _trajectory(oracle, mixer, bits, G, steps, seed):
    """Quantized BDR trajectory of one head; per step yields (prev stored
    values, S' before requantization, new codes, new scales)."""
    dk, dv = 64, 24
    w = W.Workload(80 + mixer, "bdr", mixer, 1, 1, dk, dv, G, steps, 0, W.BDR, "int8")
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=oracle.BDR)
    rng = np.random.default_rng(seed)
    S0 = (rng.standard_normal((dv, dk)) * np.exp(rng.uniform(-2, 2, (dv, 1)))).astype(np.float32)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S0, step=0)
    for t in range(steps):
        q, k, v, alpha, beta = W.step_inputs(w, t, seed=seed)
        a = alpha[0, 0] if mixer in (W.GLA, W.KDA) else np.float32([alpha[0, 0]])
        b = 0.0 if beta is None else float(beta[0, 0])
        prev = oracle.head_dequantize(c, bits, codes, scales)
        _, pre, _ = oracle.head_step(c, 0, 0, bits, codes, scales, q[0, 0], k[0, 0], v[0, 0], a,
                                     b, step=t + 1, want_pre=True)
        yield c, prev, pre, _unpack(codes, bits, dv, dk), scales.reshape(dv, dk // G).copy()


@pytest.mark.parametrize("mixer,bits,G", [(W.GDN, 4, 32), (W.GLA, 8, 64), (W.SCALAR, 4, 16),
                                          (W.KDA, 8, 32)])
def test_bdr_step_guarantees(oracle, mixer, bits, G):
    r = (1 << (bits - 1)) - 1
    reversed_by_rtn = 0
    err_rtn = err_bdr = 0.0
    n_el = 0
    for c, prev, pre, code, sc in _trajectory(oracle, mixer, bits, G, 12, 7 + mixer):
        dv, dk = pre.shape
        for i in range(dv):
            for g in range(dk // G):
                js = slice(g * G, (g + 1) * G)
                m = np.float32(np.max(np.abs(pre[i, js])))
                s_new, inv = oracle.group_scale(float(m), r)
                assert sc[i, g] == s_new
                t = [Fraction(float(x)) * Fraction(float(inv)) for x in pre[i, js]]
                rtn = _nearest_even(t)
                got = code[i, js]
                for j in range(G):
                    x, p = float(pre[i, g * G + j]), float(prev[i, g * G + j])
                    # bounded: one of the two grid neighbours of the exact value
                    assert abs(Fraction(int(got[j])) - t[j]) < 1
                    st_rtn = float(np.float32(rtn[j]) * s_new)
                    st_bdr = float(np.float32(got[j]) * s_new)
                    rev_rtn = (x > p and st_rtn < p) or (x < p and st_rtn > p)
                    # directional: no stored value moves against its update
                    assert not ((x > p and st_bdr < p) or (x < p and st_bdr > p))
                    if rev_rtn:
                        reversed_by_rtn += 1
                        assert got[j] == rtn[j] + (1 if x > p else -1)
                    else:
                        assert got[j] == rtn[j]
                    err_rtn += abs(float(Fraction(int(rtn[j])) - t[j]))
                    err_bdr += abs(float(Fraction(int(got[j])) - t[j]))
                    n_el += 1
    assert reversed_by_rtn > 0  # the trajectories do exercise the rule
    assert err_bdr > err_rtn    # larger rounding error, as the pages note
    assert n_el == 12 * 24 * 64


def test_bdr_import_rounds_to_nearest(oracle):
    """An import has no earlier stored value to move away from."""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((16, 64)).astype(np.float32)
    for bits in (4, 8):
        a = oracle.head_quantize(oracle.cfg(1, 1, 64, 16, 32, rounding=oracle.BDR), 0, 0, bits, S,
                                 step=3)
        b = oracle.head_quantize(oracle.cfg(1, 1, 64, 16, 32, rounding=oracle.RTN), 0, 0, bits, S,
                                 step=3)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
