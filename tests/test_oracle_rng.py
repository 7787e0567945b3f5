"""Pins for the counter-based random bits of the CPU reference.

The pages require stochastic rounding to be conditionally unbiased (LoReS
blog, "(3/4) Rounding"); the bits are built from three published primitives,
each pinned here by its published test vectors or by an exact property, and
the combination is checked statistically."""

import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rng_vectors.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(dict(kv.split("=", 1) for kv in line.split()[1:]) | {"kind": line.split()[0]})
    return rows


def test_splitmix64_published_vectors(oracle):
    rows = [r for r in _golden() if r["kind"] == "splitmix64"]
    assert len(rows) == 3
    x = 0
    for i, r in enumerate(rows):
        x = (x + 0x9E3779B97F4A7C15) & (2**64 - 1)
        assert oracle.splitmix64_output(x) == int(r[f"out{i}"], 16)


def test_fmix32_published_vectors(oracle):
    rows = [r for r in _golden() if r["kind"] == "murmur3_x86_32"]
    assert len(rows) == 3
    for r in rows:
        assert oracle.fmix32(int(r["seed"], 16)) == int(r["hash"], 16)


def test_fmix32_is_a_bijection_sample(oracle):
    # fmix32 is invertible (odd multipliers, xorshifts): no collisions on a sample.
    xs = np.random.default_rng(1).integers(0, 2**32, 20000, dtype=np.uint64)
    ys = {oracle.fmix32(int(x)) for x in np.unique(xs)}
    assert len(ys) == len(np.unique(xs))


M16 = 1 << 16


def _half_step(f, half):
    """The map one half of a word takes under the word step f."""
    if half == 0:
        return lambda x: f(x) & 0xFFFF
    return lambda x: f(x << 16) >> 16


def test_lcg16x2_halves_do_not_mix(oracle):
    # Each half of the next word depends on the same half of the word only.
    f = oracle.lcg16x2
    rng = np.random.default_rng(2)
    for _ in range(300):
        lo, hi, lo2, hi2 = (int(x) for x in rng.integers(0, M16, 4))
        w = f(lo | hi << 16)
        assert w & 0xFFFF == f(lo | hi2 << 16) & 0xFFFF
        assert w >> 16 == f(lo2 | hi << 16) >> 16


@pytest.mark.parametrize("half", [0, 1])
def test_lcg16x2_affine_and_full_period(oracle, half):
    # Each half is a mixed linear congruential generator x -> (a x + c) mod
    # 2^16 (a and c read off the values at 0 and 1, every other value then
    # checked against them), with c odd and a = 1 mod 4 (Hull-Dobell), and
    # its orbit from 0 visits all 2^16 values before it returns.
    step = _half_step(oracle.lcg16x2, half)
    c = step(0)
    a = (step(1) - c) % M16
    assert c % 2 == 1 and a % 4 == 1
    seen = np.zeros(M16, dtype=bool)
    x = 0
    for _ in range(M16):
        assert not seen[x]
        seen[x] = True
        y = step(x)
        assert y == (a * x + c) % M16
        x = y
    assert x == 0 and seen.all()


# Hermite constants gamma_t (exact for t <= 8).
_GAMMA = {2: (4 / 3) ** 0.5, 3: 2 ** (1 / 3), 4: 2 ** 0.5, 5: 8 ** 0.2}


def _spectral_merit(a, t):
    """nu_t / (gamma_t^(1/2) m^(1/t)): nu_t is the length of the shortest
    nonzero s with s_1 + a s_2 + ... + a^(t-1) s_t = 0 mod m (Knuth, TAOCP
    vol. 2, 3.3.4), found by exhaustive search inside the bound that the
    Hermite constant puts on it."""
    m = M16
    bound = int(np.ceil(_GAMMA[t] ** 0.5 * m ** (1 / t))) + 1
    r = np.arange(-bound, bound + 1, dtype=np.int64)
    grids = np.meshgrid(*([r] * (t - 1)), indexing="ij")
    acc = np.zeros(grids[0].shape, dtype=np.int64)
    sq = np.zeros_like(acc)
    for i, g in enumerate(grids):
        acc = (acc + pow(a, i + 1, m) * g) % m
        sq += g * g
    s1 = (-acc) % m
    s1 = np.where(s1 > m // 2, s1 - m, s1)
    n2 = sq + s1 * s1
    n2 = np.where(n2 == 0, np.iinfo(np.int64).max, n2)
    return float(np.sqrt(n2.min())) / (_GAMMA[t] ** 0.5 * m ** (1 / t))


def test_spectral_merit_reference_values():
    # Lattices worked by hand.  a = 1: the shortest dual vectors are
    # (-1, 1) and (1, -1, 0), both of length sqrt 2.  a = 257 in three
    # dimensions: 257^2 = 513 mod 2^16 and 1 - 2*257 + 513 = 0, so
    # s = (1, -2, 1) of length sqrt 6, and no s with entries in [-2, 2] is
    # shorter.
    def nu(a, t):
        return _spectral_merit(a, t) * _GAMMA[t] ** 0.5 * M16 ** (1 / t)
    assert abs(nu(1, 2) - 2 ** 0.5) < 1e-9
    assert abs(nu(1, 3) - 2 ** 0.5) < 1e-9
    assert abs(nu(257, 3) - 6 ** 0.5) < 1e-9


@pytest.mark.parametrize("half", [0, 1])
def test_lcg16x2_multipliers_pass_spectral_test(oracle, half):
    # Knuth's criterion for a good multiplier is a merit well above 0.1 in
    # each dimension; these reach at least 0.75 in dimensions 2 to 5.
    step = _half_step(oracle.lcg16x2, half)
    a = (step(1) - step(0)) % M16
    for t in (2, 3, 4, 5):
        assert _spectral_merit(a, t) >= 0.75, (hex(a), t)


def test_head_key_bits_balanced_and_avalanche(oracle):
    rng = np.random.default_rng(3)
    keys = []
    flips = []
    for _ in range(3000):
        seed = int(rng.integers(0, 2**63))
        layer, step, b, h = (int(x) for x in rng.integers(0, 1000, 4))
        k0 = oracle.head_key(seed, layer, step, b, h)
        keys.append(k0)
        # flipping one bit of one field flips about half of the key bits
        field = int(rng.integers(0, 5))
        bit = int(rng.integers(0, 10))
        args = [seed, layer, step, b, h]
        args[field] ^= 1 << bit
        flips.append(bin(k0 ^ oracle.head_key(*args)).count("1"))
    bits = np.array([[(k >> i) & 1 for i in range(32)] for k in keys])
    frac = bits.mean(axis=0)
    assert np.all(np.abs(frac - 0.5) < 0.05)
    assert abs(np.mean(flips) - 16.0) < 0.5
    assert len(set(keys)) >= len(keys) - 2


def _head_bits(oracle, key, n):
    return np.array([oracle.sr_bits(key, e) for e in range(n)], dtype=np.int64)


def test_sr_bits_uniform_and_uncorrelated(oracle):
    # 16-bit draws: uniform (chi-square on 64 bins) and no lag-1 correlation
    # between neighbouring elements, across blocks and within the block walk.
    vals = []
    for step in range(12):
        key = oracle.head_key(7, 1, step, 3, 5)
        vals.append(_head_bits(oracle, key, 4096))
    x = np.concatenate(vals)
    assert x.min() >= 0 and x.max() < 65536
    counts = np.bincount(x >> 10, minlength=64)
    expected = x.size / 64
    chi2 = np.sum((counts - expected) ** 2 / expected)
    assert chi2 < 120  # 63 dof: p ~ 3e-5
    u = (x + 0.5) / 65536.0
    for lag in (1, 2, 16):
        c = np.corrcoef(u[:-lag], u[lag:])[0, 1]
        assert abs(c) < 0.02
    # low bits are as uniform as high bits
    low = np.bincount(x & 63, minlength=64)
    assert np.sum((low - expected) ** 2 / expected) < 120


def test_sr_bits_independent_across_steps_and_heads(oracle):
    n = 2048
    a = _head_bits(oracle, oracle.head_key(0, 0, 10, 0, 0), n) / 65536.0
    b = _head_bits(oracle, oracle.head_key(0, 0, 11, 0, 0), n) / 65536.0
    c = _head_bits(oracle, oracle.head_key(0, 0, 10, 0, 1), n) / 65536.0
    d = _head_bits(oracle, oracle.head_key(0, 1, 10, 0, 0), n) / 65536.0
    for y in (b, c, d):
        assert abs(np.corrcoef(a, y)[0, 1]) < 0.08
        assert not np.array_equal(a, y)


def test_sr_bits_block_structure(oracle):
    # Elements 2p and 2p+1 share one 32-bit word: low and high halves.
    key = oracle.head_key(1, 2, 3, 4, 5)
    w0 = oracle.fmix32(key ^ 0)
    assert oracle.sr_bits(key, 0) == w0 & 0xFFFF
    assert oracle.sr_bits(key, 1) == w0 >> 16
    w1 = oracle.lcg16x2(w0)
    assert oracle.sr_bits(key, 2) == w1 & 0xFFFF
    assert oracle.sr_bits(key, 3) == w1 >> 16
    w7 = w0
    for _ in range(7):
        w7 = oracle.lcg16x2(w7)
    assert oracle.sr_bits(key, 15) == w7 >> 16
    w16 = oracle.fmix32(key ^ 1)
    assert oracle.sr_bits(key, 16) == w16 & 0xFFFF


# ---- dependence inside a 16-element block ------------------------------------------
#
# Inside a block the element pairs walk the two linear congruential streams of
# one hashed seed word: element 2p takes step p of the low-half stream, element
# 2p + 1 step p of the high-half stream.  So elements j and j + 2l (same half,
# l steps apart) carry R16 values x and A_l x + C_l (mod 2^16): fully
# dependent, not independent draws.  The pins below state that structure
# exactly and bound what it does to the stochastic-rounding decisions.


def _lcg_consts(half, lag):
    a = 0xC36D if half == 0 else 0xC23D
    A, C = 1, 0
    for _ in range(lag):
        A, C = (a * A) % M16, (a * C + 13849) % M16
    return A, C


@pytest.mark.parametrize("half", [0, 1])
def test_block_pairs_low_bits_structure(oracle, half):
    """Bit b of a half-stream has period 2^(b+1) along the block: the least
    significant bit alternates exactly between neighbouring pairs of one half
    (a and c odd), bit 1 has period 4; bits 8 and up are not periodic within a
    block (8 pairs)."""
    rng = np.random.default_rng(5 + half)
    keys = rng.integers(0, 2**32, 200, dtype=np.uint64)
    for key in keys:
        for blk in (0, 7, 12345):
            r = [oracle.sr_bits(int(key), 16 * blk + 2 * p + half) for p in range(8)]
            lsb = [x & 1 for x in r]
            assert all(lsb[p] != lsb[p + 1] for p in range(7))  # exact alternation
            b1 = [(x >> 1) & 1 for x in r]
            assert all(b1[p] == b1[p + 4] for p in range(4))    # period 4
            for lag in range(1, 8):  # the affine relation inside the block
                A, C = _lcg_consts(half, lag)
                assert all(r[p + lag] == (A * r[p] + C) % M16 for p in range(8 - lag))


def _joint_deviation(A, C, grid=65):
    """max over threshold pairs (T1, T2) of |P(x >= T1 and y >= T2) - P(x >= T1) P(y >= T2)|
    for x uniform on [0, 2^16) and y = (A x + C) mod 2^16, counted exactly."""
    x = np.arange(M16, dtype=np.int64)
    y = (A * x + C) % M16
    T = np.linspace(0, M16, grid).astype(np.int64)
    # counts of (x >= T1, y >= T2) via a 2-D histogram on the threshold grid
    ix = np.searchsorted(T, x, side="right") - 1
    iy = np.searchsorted(T, y, side="right") - 1
    H = np.zeros((grid, grid), np.int64)
    np.add.at(H, (ix, iy), 1)
    # N[a, b] = #{x >= T[a], y >= T[b]}: reverse cumulative sums
    N = H[::-1, ::-1].cumsum(0).cumsum(1)[::-1, ::-1]
    px = (M16 - T) / M16
    return float(np.max(np.abs(N / M16 - np.outer(px, px))))


@pytest.mark.parametrize("half", [0, 1])
def test_block_pairs_sr_decisions_nearly_independent(half):
    """Two elements of one block and one half, l pairs apart, round up when
    their R16 values pass thresholds T1 and T2 set by their fractional parts.
    Counted exactly over all 2^16 values of the first, the joint probability
    of rounding both up differs from the product of the marginals by less
    than 1e-3 (measured: at most 1.7e-4) for every l = 1..7 and every pair of
    thresholds on a 1/64 grid: the 2-D lattice of a spectrally tested
    multiplier."""
    worst = max(_joint_deviation(*_lcg_consts(half, lag)) for lag in range(1, 8))
    assert worst < 1e-3, worst


def test_block_dependence_leaves_readout_error_variance(oracle):
    """Readout-error variance of a stochastically rounded head (unit q): the
    reference's random bits against independent uniform draws on the same
    2^-16 grid, over 1500 quantization events each.  The within-block
    dependence changes the variance by less than the sampling noise (about
    4 %): ratio within [0.92, 1.08]."""
    rng = np.random.default_rng(77)
    dv, dk, G, bits = 16, 128, 32, 4
    c = oracle.cfg(1, 1, dk, dv, G, rounding=1, seed=3)
    S = rng.standard_normal((dv, dk)).astype(np.float32)
    q = rng.standard_normal(dk)
    q /= np.linalg.norm(q)
    r = 2 ** (bits - 1) - 1
    inv = np.zeros((dv, dk))
    sc = np.zeros((dv, dk))
    for i in range(dv):
        for g in range(dk // G):
            m = float(np.abs(S[i, g * G:(g + 1) * G]).max())
            s, iv = oracle.group_scale(m, r)
            inv[i, g * G:(g + 1) * G] = float(iv)
            sc[i, g * G:(g + 1) * G] = float(s)
    t = S.astype(np.float64) * inv
    x = np.rint(t * 65536) / 65536  # the 2^-16 pre-rounding of 4-bit codes
    exact = S.astype(np.float64) @ q
    n = 1500
    err_ref, err_ind = [], []
    for step in range(n):
        codes, _, _ = oracle.head_quantize(c, 0, 0, bits, S, step)
        v = np.empty(codes.size * 2, np.int64)
        v[0::2], v[1::2] = codes & 0xF, codes >> 4
        v[v >= 8] -= 16
        err_ref.append((v.reshape(dv, dk) * sc) @ q - exact)
        u = rng.integers(0, 65536, (dv, dk)) / 65536
        ci = np.clip(np.floor(x + u), -r, r)
        err_ind.append((ci * sc) @ q - exact)
    var_ref = np.var(np.array(err_ref), axis=0).mean()
    var_ind = np.var(np.array(err_ind), axis=0).mean()
    assert 0.92 < var_ref / var_ind < 1.08, (var_ref, var_ind)
