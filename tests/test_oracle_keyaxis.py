"""Pins for key-axis scale groups in the CPU reference.

LoReS blog, "Scale grouping" (1/4): the state has two feature axes and the
page compares value-axis groups (a scale per value row, the default) with
key-axis groups (a scale per key column, C_j = max_i |S_ij| in Prop.
"per-channel readout error").  Key-axis groups of G value rows are pinned to
the value-axis quantizer of the transposed state, to the proposition's
key-axis error formula, and to the update of the stored state."""

import numpy as np
import pytest

import workloads as W

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2


def _unpack(codes, bits, rows, cols):
    if bits == 8:
        return codes.view(np.int8).astype(np.int64).reshape(rows, cols)
    x = np.empty(codes.size * 2, np.int64)
    x[0::2], x[1::2] = codes & 0xF, codes >> 4
    x[x >= 8] -= 16
    return x.reshape(rows, cols)


def _state(rng, dv, dk):
    return (rng.standard_normal((dv, dk)) * np.exp(rng.uniform(-3, 3, (dv, 1)))
            * np.exp(rng.uniform(-1, 1, (1, dk)))).astype(np.float32)


def _unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [16, 32, 64])
@pytest.mark.parametrize("rounding", [RTN, BDR])
def test_key_axis_is_value_axis_of_the_transpose(oracle, bits, G, rounding):
    """A key-axis group of S is a value-axis group of S^T (nearest rounding;
    an import under BDR rounds to nearest too)."""
    rng = np.random.default_rng(300 + bits + G)
    dv, dk = 128, 64
    S = _state(rng, dv, dk)
    S[G:2 * G, 5] = 0.0  # an all-zero key-axis group
    ck = oracle.cfg(1, 1, dk, dv, G, rounding=rounding, axis=oracle.KEY_AXIS)
    cv = oracle.cfg(1, 1, dv, dk, G, rounding=RTN)
    kc, ks, _ = oracle.head_quantize(ck, 0, 0, bits, S, step=2)
    vc, vs, _ = oracle.head_quantize(cv, 0, 0, bits, np.ascontiguousarray(S.T), step=2)
    assert np.array_equal(_unpack(kc, bits, dv, dk), _unpack(vc, bits, dk, dv).T)
    assert np.array_equal(ks.reshape(dv // G, dk), vs.reshape(dk, dv // G).T)
    Sk = oracle.head_dequantize(ck, bits, kc, ks)
    Sv = oracle.head_dequantize(cv, bits, vc, vs)
    assert np.array_equal(Sk, Sv.T)


@pytest.mark.parametrize("bits", [4, 8])
def test_key_axis_readout_error_matches_the_proposition(oracle, bits):
    """Prop. "per-channel readout error", key-axis line: with one scale per
    key column (G = dv), E[e_i^2] = sum_j q_j^2 C_j^2 / (12 r^2), the same
    for every channel.  The proposition assumes errors uniform within half a
    step, so the states spread their magnitudes over key columns only."""
    rng = np.random.default_rng(320 + bits)
    dk = dv = 128
    r = 2 ** (bits - 1) - 1
    ck = oracle.cfg(1, 1, dk, dv, dv, rounding=RTN, axis=oracle.KEY_AXIS)
    ratios = []
    for head in range(48):
        S = (rng.standard_normal((dv, dk)) * np.exp(rng.uniform(-2, 2, (1, dk)))).astype(np.float32)
        q = _unit(rng, dk).astype(np.float64)
        codes, scales, _ = oracle.head_quantize(ck, 0, head, bits, S, step=0)
        e = (oracle.head_dequantize(ck, bits, codes, scales).astype(np.float64) - S) @ q
        C = np.abs(S).max(axis=0).astype(np.float64)
        ratios.append(e**2 / (np.sum(q**2 * C**2) / (12 * r**2)))
    ratio = np.concatenate(ratios).mean()
    assert abs(ratio - 1.0) < 0.05, ratio


@pytest.mark.parametrize("bits", [4, 8])
def test_key_axis_hurts_small_rows(oracle, bits):
    """The same section's reading of the proposition: under key-axis groups
    large entries in one row set coarse steps for the other rows, so value
    rows of small magnitude read out far larger errors than under value-axis
    groups."""
    rng = np.random.default_rng(330 + bits)
    dk = dv = 128
    ck = oracle.cfg(1, 1, dk, dv, dv, rounding=RTN, axis=oracle.KEY_AXIS)
    cv = oracle.cfg(1, 1, dk, dv, dk, rounding=RTN)
    small_k, small_v = [], []
    for head in range(16):
        S = _state(rng, dv, dk)
        q = _unit(rng, dk).astype(np.float64)
        small = np.argsort(np.abs(S).max(axis=1))[:16]
        for c, out in ((ck, small_k), (cv, small_v)):
            codes, scales, _ = oracle.head_quantize(c, 0, head, bits, S, step=0)
            e = (oracle.head_dequantize(c, bits, codes, scales).astype(np.float64) - S) @ q
            out.append(e[small] ** 2)
    assert np.mean(small_k) > 10 * np.mean(small_v)


@pytest.mark.parametrize("mixer", [GDN, GLA, SCALAR, KDA])
@pytest.mark.parametrize("rounding", [SR, BDR])
def test_key_axis_step_updates_the_stored_state(oracle, mixer, rounding):
    """The step reads the stored state through the key-axis scales, updates
    it in full precision (float64 matrix form) and requantizes every key
    column group from the updated state."""
    rng = np.random.default_rng(340 + 4 * mixer + rounding)
    dk, dv, G, bits = 64, 48, 16, 4 + 4 * (mixer % 2)
    r = 2 ** (bits - 1) - 1
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=rounding, seed=9, axis=oracle.KEY_AXIS)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bits, _state(rng, dv, dk), step=0)
    for t in range(1, 5):
        prev = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        q, k = _unit(rng, dk), _unit(rng, dk)
        v = rng.standard_normal(dv).astype(np.float32)
        k64, v64 = k.astype(np.float64), v.astype(np.float64)
        beta = float(np.float32(rng.uniform(0.1, 1.5))) if mixer != GLA else 0.0
        if mixer in (GLA, KDA):
            alpha = rng.uniform(0.8, 1.0, dk).astype(np.float32)
            D = prev @ np.diag(alpha.astype(np.float64))
        else:
            alpha = np.float32([rng.uniform(0.8, 1.0)])
            D = prev * float(alpha[0])
        if mixer in (GDN, KDA):
            want = D @ (np.eye(dk) - beta * np.outer(k64, k64)) + beta * np.outer(v64, k64)
        elif mixer == GLA:
            want = D + np.outer(v64, k64)
        else:
            want = D + beta * np.outer(v64, k64)
        o, pre, _ = oracle.head_step(c, 0, 0, bits, codes, scales, q, k, v, alpha, beta, step=t,
                                     want_pre=True)
        tol = 2e-6 * max(1.0, np.abs(want).max())
        assert np.max(np.abs(pre - want)) <= tol
        assert np.max(np.abs(o - want @ q.astype(np.float64))) <= 8 * tol
        # new scales: absmax over each group of G rows of one column, divided by r
        m = np.abs(pre).reshape(dv // G, G, dk).max(axis=1)
        assert np.array_equal(scales.reshape(dv // G, dk), (m / np.float32(r)).astype(np.float32))
        got = oracle.head_dequantize(c, bits, codes, scales).astype(np.float64)
        step_size = np.repeat(scales.reshape(dv // G, dk), G, axis=0).astype(np.float64)
        assert np.all(np.abs(got - pre) <= step_size * (1 + 2**-10))
        if rounding == BDR:  # no stored value moved against its update
            p, x = prev.astype(np.float32), pre
            st = got.astype(np.float32)
            assert not np.any(((x > p) & (st < p)) | ((x < p) & (st > p)))


@pytest.mark.parametrize("dv,G", [(32, 16), (128, 128)])
def test_key_axis_batch_wrappers_match_per_head(oracle, dv, G):
    """Per-head scale blocks of (dv/G)*dk floats, also when G exceeds dk."""
    rng = np.random.default_rng(360 + G)
    B, H, dk = 2, 3, 64
    hb = np.array([4, 8, 4], np.uint8)
    c = oracle.cfg(B, H, dk, dv, G, mixer=GDN, rounding=SR, seed=3, axis=oracle.KEY_AXIS)
    S = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
    codes, scales = oracle.quantize(c, hb, S, 0)
    assert scales.shape == (B, H, dv // G, dk)
    q = rng.standard_normal((B, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, dv)).astype(np.float32)
    alpha = rng.uniform(0.5, 1, (B, H)).astype(np.float32)
    beta = rng.uniform(0, 1, (B, H)).astype(np.float32)
    c2, s2 = codes.copy(), scales.copy()
    o = oracle.step(c, hb, c2, s2, q, k, v, alpha, beta, 1)
    for b in range(B):
        for h in range(H):
            off = oracle.head_offset(c, b, h, hb)
            n = dv * dk * int(hb[h]) // 8
            hc, hs = codes[off:off + n].copy(), scales[b, h].copy()
            oh, _, _ = oracle.head_step(c, b, h, int(hb[h]), hc, hs, q[b, h], k[b, h], v[b, h],
                                        np.float32([alpha[b, h]]), float(beta[b, h]), step=1)
            assert np.array_equal(hc, c2[off:off + n]) and np.array_equal(hs, s2[b, h])
            assert np.array_equal(oh, o[b, h])
