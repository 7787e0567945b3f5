"""Pins for the reference's threshold distance and the parity exemption rule.

The parity contract lets two quantizer implementations differ by one code
only where the exact pre-rounding value t = S'*inv lies within 1e-6 code
units of a point where the code changes.  The reference reports that
distance per element; here it is checked against the code function itself,
evaluated in exact rational arithmetic from its definitions:
  * round to nearest (LoReS blog, "(3/4) Rounding", RTN): rint(t), ties to
    even, clamped to [-r, r];
  * stochastic rounding (same section; its random-bit form as the reference
    defines it): floor((RN(t 2^f) 2^(16-f) + r16) / 2^16), f = 16 for 4-bit
    and 15 for 8-bit codes, clamped to [-r, r].
Then mismatches are planted next to exact thresholds and far from them, and
the rule must exempt exactly the near ones."""

from fractions import Fraction

import numpy as np
import pytest

from exemption import NEAR, ParityError, classify

RTN, SR = 0, 1


def _rn_even(x: Fraction) -> int:
    """Nearest integer, ties to even, exactly."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def _code(t: Fraction, stochastic: bool, r16: int, bits: int) -> int:
    r = 2 ** (bits - 1) - 1
    if stochastic:
        f = 16 if bits == 4 else 15
        n = _rn_even(t * 2**f)
        c = (n * 2 ** (16 - f) + r16) // 2**16
    else:
        c = _rn_even(t)
    return max(-r, min(r, c))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("stochastic", [False, True])
def test_distance_brackets_the_code_change(oracle, bits, stochastic):
    """Inside the reported distance the code is constant; just beyond it, on
    one side, it changes (the nearest change point is at that distance)."""
    rng = np.random.default_rng(300 + bits + 10 * stochastic)
    r = 2 ** (bits - 1) - 1
    for trial in range(1500):
        m = np.float32(np.exp(rng.uniform(-8, 8)))
        _, inv = oracle.group_scale(float(m), r)
        x = np.float32(m * rng.uniform(-1, 1))
        if trial % 5 == 0:  # some at the group max
            x = np.float32(m if trial % 10 == 0 else -m)
        r16 = int(rng.integers(0, 65536))
        d = oracle.threshold_distance(float(x), float(inv), stochastic, r16, bits)
        t = Fraction(float(x)) * Fraction(float(inv))
        assert 0.0 <= d <= 1.0
        c0 = _code(t, stochastic, r16, bits)
        D = Fraction(d)
        inside = [t - D * Fraction(999, 1000), t + D * Fraction(999, 1000)]
        assert all(_code(p, stochastic, r16, bits) == c0 for p in inside), (x, inv, r16, d)
        beyond = [t - D * Fraction(1001, 1000) - Fraction(1, 2**60),
                  t + D * Fraction(1001, 1000) + Fraction(1, 2**60)]
        assert any(_code(p, stochastic, r16, bits) != c0 for p in beyond), (x, inv, r16, d)


def _threshold(stochastic: bool, n: int, r16: int, bits: int) -> float:
    """An exact threshold t (a float) where the code steps from n - 1 to n."""
    if not stochastic:
        return float(np.float32(n - 0.5))
    c = Fraction(r16 | 1) if bits == 8 else Fraction(2 * r16 + 1, 2)
    tau = Fraction(n) - c / 2**16
    assert Fraction(float(np.float32(float(tau)))) == tau  # representable
    return float(tau)


@pytest.mark.parametrize("bits,rounding", [(4, RTN), (8, RTN), (4, SR), (8, SR)])
def test_exemption_takes_exactly_the_near_mismatches(oracle, bits, rounding):
    """A head whose groups each have absmax r (so s = 1 and t = S' exactly),
    with elements placed on exact code thresholds, a few ulps from them, and
    far from them.  Codes flipped by one at near elements are exempted; a
    single far flip fails the comparison."""
    r = 2 ** (bits - 1) - 1
    dv, dk, G = 8, 64, 32
    seed, layer, step, b, h = 5, 2, 3, 0, 0
    c = oracle.cfg(1, 1, dk, dv, G, rounding=rounding, seed=seed, layer=layer)
    key = oracle.head_key(seed, layer, step, b, h)
    stochastic = rounding == SR
    rng = np.random.default_rng(77 + bits + rounding)
    S = np.float32(rng.uniform(-0.9, 0.9, (dv, dk)) * (r - 1))
    near, far = [], []
    for i in range(dv):
        for g in range(dk // G):
            S[i, g * G] = np.float32(r if (i + g) % 2 else -r)  # the group max: inv = 1
            for k in range(1, G):
                e = i * dk + g * G + k
                if k % 3 == 0:
                    continue  # keep some ordinary elements
                n = int(rng.integers(-r + 2 if bits == 4 else 1, r - 1 if bits == 4 else 4))
                n = n if bits == 4 or k % 2 else -n
                tau = _threshold(stochastic, n, oracle.sr_bits(key, e) & 0xFFFF, bits)
                kind = k % 5
                x = np.float32(tau)
                if kind <= 2:  # on the threshold or a few ulps above it
                    for _ in range(kind):
                        x = np.nextafter(x, np.float32(np.inf))
                else:  # clearly away from it
                    x = np.float32(tau + (0.003 if kind == 3 else -0.2))
                S[i, g * G + k] = x
                (near if abs(float(x) - tau) < NEAR else far).append(e)
    assert all(oracle.group_scale(float(np.abs(S[i, g * G:(g + 1) * G]).max()), r)
               == (1.0, 1.0) for i in range(dv) for g in range(dk // G))
    codes, scales, tdist = oracle.head_quantize(c, b, h, bits, S, step, want_tdist=True)
    ref = _unpack(codes, bits, dv, dk).ravel()
    td = tdist.ravel()
    assert len(near) > 20 and len(far) > 20
    assert np.all(td[near] < NEAR) and np.all(td[far] >= NEAR)
    gpu = ref.copy()
    flip = np.where(ref[near] < r, 1, -1)
    gpu[near] += flip
    got = classify(gpu, ref, td, "planted near")
    assert sorted(got.tolist()) == sorted(near)
    for e in far[:5]:
        g2 = gpu.copy()
        g2[e] += 1 if ref[e] < r else -1
        with pytest.raises(ParityError):
            classify(g2, ref, td, "planted far")
    # two codes apart is never exempt, even on a threshold
    g3 = ref.copy()
    g3[near[0]] += 2 if ref[near[0]] < r - 1 else -2
    with pytest.raises(ParityError):
        classify(g3, ref, td, "two apart")


def test_exemption_on_ordinary_states_is_rare(oracle):
    """On a random state almost no element is near a threshold: the rate the
    contract allows (1e-5) is not reached by chance."""
    rng = np.random.default_rng(91)
    dv, dk, G = 128, 128, 32
    for bits, rounding in ((4, SR), (8, SR), (4, RTN), (8, RTN)):
        c = oracle.cfg(1, 1, dk, dv, G, rounding=rounding, seed=1)
        S = rng.standard_normal((dv, dk)).astype(np.float32)
        _, _, td = oracle.head_quantize(c, 0, 0, bits, S, 7, want_tdist=True)
        assert np.count_nonzero(td < NEAR) <= 2


def _unpack(codes, bits, dv, dk):
    if bits == 8:
        return codes.view(np.int8).astype(np.int32).reshape(dv, dk)
    x = np.empty(codes.size * 2, np.int32)
    x[0::2], x[1::2] = codes & 0xF, codes >> 4
    x[x >= 8] -= 16
    return x.reshape(dv, dk)
