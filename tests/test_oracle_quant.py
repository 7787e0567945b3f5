"""Pins for the state quantizer of the CPU reference.

Symmetric absmax quantizer with r = 2^(b-1) - 1 and s = |S_G|_inf / r (LoReS
blog, Prop. "per-channel readout error"; 4/4 animation details), value-axis
(row) groups (1/4), round-to-nearest and stochastic rounding (3/4), INT4 codes
packed two per byte."""

import math
from fractions import Fraction

import numpy as np
import pytest

GDN, GLA, SCALAR = 0, 1, 2
RTN, SR = 0, 1


def _unpack(codes: np.ndarray, bits: int, dv: int, dk: int) -> np.ndarray:
    """Independent numpy decoding of the code layout."""
    if bits == 8:
        return codes.view(np.int8).astype(np.int32).reshape(dv, dk)
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    x = np.empty(codes.size * 2, np.int32)
    x[0::2], x[1::2] = lo, hi
    x[x >= 8] -= 16
    return x.reshape(dv, dk)


def _state(rng, dv, dk, spread=True):
    S = rng.standard_normal((dv, dk))
    if spread:  # rows of very different magnitude, as value channels are
        S *= np.exp(rng.uniform(-3, 3, (dv, 1)))
    return S.astype(np.float32)


def test_group_scale_exact(oracle):
    rng = np.random.default_rng(50)
    ms = list(np.abs(rng.standard_normal(300)).astype(np.float32))
    ms += [np.float32(x) for x in (1.0, 127.0, 7.0, 1e-30, 3e-38, 1e-44, 3.0e38, 0.1)]
    for r in (7, 127):
        for m in ms:
            s, inv = oracle.group_scale(float(m), r)
            assert s == np.float32(m) / np.float32(r)  # IEEE division
            M, R = Fraction(float(m)), Fraction(r)
            assert Fraction(float(inv)) * M <= R
            if inv < np.finfo(np.float32).max:
                nxt = np.nextafter(inv, np.float32(np.inf))
                assert Fraction(float(nxt)) * M > R  # largest such float
    assert oracle.group_scale(0.0, 7) == (0.0, 0.0)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [16, 32, 64])
def test_rtn_is_nearest_grid_point(oracle, bits, G):
    rng = np.random.default_rng(51 + bits + G)
    dv, dk = 24, 64
    c = oracle.cfg(1, 1, dk, dv, G, rounding=RTN)
    S = _state(rng, dv, dk)
    S[3, :G] = 0.0  # an all-zero group
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S, step=0)
    n = _unpack(codes, bits, dv, dk)
    r = 2 ** (bits - 1) - 1
    sc = scales.reshape(dv, dk // G)
    for i in range(dv):
        for g in range(dk // G):
            seg = S[i, g * G:(g + 1) * G]
            m = np.abs(seg).max()
            s, inv = oracle.group_scale(float(m), r)
            assert sc[i, g] == s
            t = seg.astype(np.float64) * np.float64(inv)  # exact products
            cands = np.arange(-r, r + 1, dtype=np.float64)
            dist = np.abs(cands[None, :] - t[:, None])  # exact in float64
            dmin = dist.min(axis=1, keepdims=True)
            tie_even = (dist == dmin) & (cands[None, :] % 2 == 0)
            best = np.where(tie_even.any(axis=1), cands[np.argmax(tie_even, axis=1)],
                            cands[np.argmin(dist, axis=1)])
            assert np.array_equal(n[i, g * G:(g + 1) * G], best.astype(np.int32))
            # RTN error bound: half a step, with FP slack
            err = np.abs(n[i, g * G:(g + 1) * G] * np.float64(s) - seg.astype(np.float64))
            assert np.all(err <= np.float64(s) * (0.5 + 2**-14) + 1e-45)
            if m > 0:
                assert np.abs(n[i, g * G:(g + 1) * G]).max() == r
            else:
                assert np.all(n[i, g * G:(g + 1) * G] == 0)


@pytest.mark.parametrize("bits", [4, 8])
def test_rtn_idempotent(oracle, bits):
    rng = np.random.default_rng(52)
    dv, dk, G = 16, 64, 32
    c = oracle.cfg(1, 1, dk, dv, G, rounding=RTN)
    S = _state(rng, dv, dk)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S, step=0)
    Sq = oracle.head_dequantize(c, bits, codes, scales)
    codes2, scales2, _ = oracle.head_quantize(c, 0, 0, bits, Sq, step=5)
    assert np.array_equal(codes, codes2)
    # scales may move by one ulp (the double rounding of r*s)
    assert np.all(np.abs(scales2.view(np.int32) - scales.view(np.int32)) <= 1)


def test_sr_exhaustive_expectation(oracle):
    """Over all 65536 draws R, the stochastic-rounding code averages exactly to
    x*inv rounded to the nearest multiple of 2^-f (f = 16 for INT4, 15 for
    INT8; ties to even), which is within 2^-(f+1) of x*inv: conditional
    unbiasedness (3/4) up to that fixed resolution.  Exact rational
    arithmetic, independent of the oracle's formula."""
    rng = np.random.default_rng(53)
    R = np.arange(65536)
    for bits, f in ((4, 16), (8, 15)):
        r = 2 ** (bits - 1) - 1
        for i in range(8):
            m = np.float32(abs(rng.standard_normal()) + 0.1)
            s, inv = oracle.group_scale(float(m), r)
            x = np.float32(rng.uniform(-1, 1) * m) if i else np.float32(m)
            t = Fraction(float(x)) * Fraction(float(inv))
            tf = Fraction(round(t * 2 ** f), 2 ** f)  # Python's round: ties to even
            assert abs(tf - t) <= Fraction(1, 2 ** (f + 1))
            vals = np.array([oracle.round_sr(float(x), float(inv), int(rr), bits) for rr in R])
            lo = math.floor(tf)
            assert set(np.unique(vals).tolist()) <= {lo, lo + 1}
            assert Fraction(int(vals.sum()), 65536) == tf
            assert abs(vals).max() <= r


def test_sr_threshold_and_ties(oracle):
    """Hand cases of the SR definition: inv = 1 and x on the 2^-16 grid give
    code = floor(x + R/2^16) exactly; the first rounding to 2^-f is
    half-to-even (x = 2^-17 rounds to 0 for INT4, so every draw gives 0)."""
    # x = 0.25: R < 49152 -> 0, R >= 49152 -> 1
    assert oracle.round_sr(0.25, 1.0, 49151, 4) == 0
    assert oracle.round_sr(0.25, 1.0, 49152, 4) == 1
    # negative: x = -0.25 -> floor(-0.25 + R/2^16): R < 16384 -> -1
    assert oracle.round_sr(-0.25, 1.0, 16383, 4) == -1
    assert oracle.round_sr(-0.25, 1.0, 16384, 4) == 0
    # ties at the 2^-16 (INT4) grid: 2^-17 -> 0, 3*2^-17 -> 2^-15 (even)
    assert oracle.round_sr(2.0 ** -17, 1.0, 65535, 4) == 0
    assert oracle.round_sr(3 * 2.0 ** -17, 1.0, 65534, 4) == 1
    assert oracle.round_sr(3 * 2.0 ** -17, 1.0, 65533, 4) == 0
    # INT8 rounds to the 2^-15 grid first: 2^-16 -> 0 (tie to even), 3*2^-16 -> 2^-14
    assert oracle.round_sr(2.0 ** -16, 1.0, 65535, 8) == 0
    assert oracle.round_sr(3 * 2.0 ** -16, 1.0, 65532, 8) == 1
    assert oracle.round_sr(3 * 2.0 ** -16, 1.0, 65531, 8) == 0
    # the ends of the range stay inside [-r, r]
    assert oracle.round_sr(7.0, 1.0, 65535, 4) == 7
    assert oracle.round_sr(-127.0, 1.0, 0, 8) == -127


@pytest.mark.parametrize("bits", [4, 8])
def test_sr_unbiased_through_real_hash(oracle, bits):
    """1e5 independent quantizations (distinct step counters) of one state: the
    mean code equals S*inv per element within 5 standard errors."""
    rng = np.random.default_rng(54)
    dv, dk, G = 2, 32, 32
    c = oracle.cfg(1, 1, dk, dv, G, rounding=SR, seed=99)
    S = _state(rng, dv, dk, spread=False)
    r = 2 ** (bits - 1) - 1
    N = 100_000
    acc = np.zeros((dv, dk))
    for t in range(N):
        codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, S, step=t)
        acc += _unpack(codes, bits, dv, dk)
    mean = acc / N
    _, scales, _ = oracle.head_quantize(c, 0, 0, bits, S, step=0)
    inv = np.array([[oracle.group_scale(float(np.abs(S[i]).max()), r)[1]] for i in range(dv)])
    t = S.astype(np.float64) * inv
    # exact expectation on the 2^-16 draw grid: P(up) = #{R : R/2^16 >= 1 - f} / 2^16
    f = t - np.floor(t)
    p_up = (65536 - np.ceil(65536 * (1 - f))) / 65536
    expect = np.floor(t) + p_up
    assert np.all(np.abs(expect - t) <= 2.0**-16)  # the grid bias, at most one draw step
    se = np.sqrt(p_up * (1 - p_up) / N)
    assert np.all(np.abs(mean - expect) <= 5 * se + 5.0 / N)


@pytest.mark.parametrize("bits", [4, 8])
def test_sr_step_counter_and_determinism(oracle, bits):
    rng = np.random.default_rng(55)
    dv, dk, G = 8, 64, 32
    c = oracle.cfg(1, 1, dk, dv, G, rounding=SR, seed=5, layer=2)
    S = _state(rng, dv, dk)
    a = oracle.head_quantize(c, 3, 4, bits, S, step=7)
    b = oracle.head_quantize(c, 3, 4, bits, S, step=7)
    d = oracle.head_quantize(c, 3, 4, bits, S, step=8)
    e = oracle.head_quantize(c, 3, 5, bits, S, step=7)
    assert np.array_equal(a[0], b[0])
    assert not np.array_equal(a[0], d[0])
    assert not np.array_equal(a[0], e[0])
    assert np.array_equal(a[1], d[1])  # scales do not depend on the draws


def test_int4_nibble_layout(oracle):
    dv, dk = 2, 16
    buf = np.zeros(dv * dk // 2, np.uint8)
    from oracle import lib, _ptr
    vals = np.arange(-8, 8).tolist() * 2
    for e, v in enumerate(vals):
        lib().oracle_set_code(_ptr(buf), 4, e, v)
    # even element in the low nibble, two's complement
    assert buf[0] == ((-8 & 0xF) | ((-7 & 0xF) << 4))
    assert np.array_equal(_unpack(buf, 4, dv, dk).ravel(), np.array(vals))
    for e, v in enumerate(vals):
        assert oracle.get_code(buf, 4, e) == v


def test_head_offsets_mixed_bits(oracle):
    c = oracle.cfg(3, 5, 64, 32, 32)
    hb = np.array([4, 8, 8, 4, 4], np.uint8)
    sizes = 32 * 64 * hb.astype(int) // 8
    per_b = sizes.sum()
    assert oracle.codes_bytes(c, hb) == 3 * per_b
    for b in range(3):
        for h in range(5):
            assert oracle.head_offset(c, b, h, hb) == b * per_b + sizes[:h].sum()


def test_bits_by_decay_rules(oracle):
    ret = np.array([0.95, 0.995, 0.991, 0.99, 0.90, 0.999], np.float32)
    out = oracle.bits_by_decay(ret, 0, 0.99)
    assert out.tolist() == [4, 8, 8, 4, 4, 8]
    # rank: half the heads, largest retention first, ties to the lower index
    ret = np.array([0.5, 0.9, 0.7, 0.9, 0.1, 0.7], np.float32)
    assert oracle.bits_by_decay(ret, 1, 0.5).tolist() == [4, 8, 8, 8, 4, 4]
    assert oracle.bits_by_decay(ret, 1, 0.0).tolist() == [4] * 6
    assert oracle.bits_by_decay(ret, 1, 1.0).tolist() == [8] * 6
    rng = np.random.default_rng(56)
    for _ in range(50):
        ret = rng.choice([0.1, 0.2, 0.3, 0.4], 16).astype(np.float32)
        out = oracle.bits_by_decay(ret, 1, 0.5)
        assert (out == 8).sum() == 8
        order = sorted(range(16), key=lambda h: (-ret[h], h))
        assert set(np.nonzero(out == 8)[0]) == set(order[:8])


@pytest.mark.parametrize("bits", [4, 8])
def test_rtn_exact_ties_go_to_even(oracle, bits):
    """A group whose absmax is r itself has inv = 1 exactly, so half-integer
    states are exact ties: round-half-to-even decides them."""
    r = 2 ** (bits - 1) - 1
    dk, G = 16, 16
    c = oracle.cfg(1, 1, dk, 1, G, rounding=RTN)
    row = np.array([r, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -3.5, 4.5, 0, 0, 0, 0, 0, 0],
                   np.float32)
    if bits == 4:
        row[9] = 0.25
    assert oracle.group_scale(float(r), r) == (1.0, 1.0)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, row, step=0)
    got = _unpack(codes, bits, 1, dk).ravel()
    want = [r, 0, 2, 2, 0, -2, -2, 4, -4, 4 if bits == 8 else 0, 0, 0, 0, 0, 0, 0]
    assert got.tolist() == want
