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


def _gf2_matrix(f):
    """32x32 matrix over GF(2) of a linear map on 32-bit words (column j = f(e_j))."""
    M = np.zeros((32, 32), dtype=np.uint8)
    for j in range(32):
        y = f(1 << j)
        for i in range(32):
            M[i, j] = (y >> i) & 1
    return M


def _matmul2(A, B):
    return (A.astype(np.int64) @ B.astype(np.int64) % 2).astype(np.uint8)


def _matpow2(A, e):
    R = np.eye(32, dtype=np.uint8)
    while e:
        if e & 1:
            R = _matmul2(R, A)
        A = _matmul2(A, A)
        e >>= 1
    return R


def test_xorshift32_linear_full_period(oracle):
    # Marsaglia (2003): with a valid shift triple the xorshift32 map has
    # period 2^32 - 1 on nonzero words, i.e. its GF(2) matrix T has order
    # exactly 2^32 - 1 = 3*5*17*257*65537.  A wrong shift amount or direction
    # breaks linearity or the order.
    f = oracle.xorshift32
    rng = np.random.default_rng(2)
    for _ in range(200):
        a, b = (int(x) for x in rng.integers(0, 2**32, 2, dtype=np.uint64))
        assert f(a ^ b) == f(a) ^ f(b)
    T = _gf2_matrix(f)
    I = np.eye(32, dtype=np.uint8)
    n = 2**32 - 1
    assert np.array_equal(_matpow2(T, n), I)
    for p in (3, 5, 17, 257, 65537):
        assert not np.array_equal(_matpow2(T, n // p), I)


def test_xorshift32_fixed_point_zero(oracle):
    assert oracle.xorshift32(0) == 0


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
    # between neighbouring elements, across blocks and within the xorshift walk.
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
    w0 = oracle.fmix32(key ^ 0) or 1
    assert oracle.sr_bits(key, 0) == w0 & 0xFFFF
    assert oracle.sr_bits(key, 1) == w0 >> 16
    w1 = oracle.xorshift32(w0)
    assert oracle.sr_bits(key, 2) == w1 & 0xFFFF
    w16 = oracle.fmix32(key ^ 1) or 1
    assert oracle.sr_bits(key, 16) == w16 & 0xFFFF
