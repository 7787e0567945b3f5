"""Pins for per-channel bit widths in the CPU reference.

LoReS blog, "Mixed precision" (2/4): decay attenuates quantization error, so
the slowest-decaying heads or channels get more bits.  Channels here are key
columns, allocated per block of 16 (the unit one lane of the kernels owns);
a row stores its blocks in column order, 16 bytes per INT8 block and 8 per
INT4 block.  A scale group never mixes widths, so a mixed head quantizes
exactly as the uniform INT8 and INT4 quantizations of the same state, block
by block; pinned here with an independent decoder of the byte layout, and
the allocation itself is pinned to the proposition it serves: slow channels
with more bits accumulate less error than fast ones with more bits."""

import numpy as np
import pytest

import workloads as W

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2


def _decode_mixed(codes, bb, dv, dk):
    """Independent numpy decoding of the mixed-width row layout."""
    row_bytes = int(np.sum(2 * bb.astype(np.int64)))
    rows = codes.reshape(dv, row_bytes)
    out = np.empty((dv, dk), np.int64)
    off = 0
    for q, bits in enumerate(bb):
        if bits == 8:
            out[:, 16 * q:16 * q + 16] = rows[:, off:off + 16].view(np.int8)
            off += 16
        else:
            blk = rows[:, off:off + 8]
            x = np.empty((dv, 16), np.int64)
            x[:, 0::2], x[:, 1::2] = blk & 0xF, blk >> 4
            x[x >= 8] -= 16
            out[:, 16 * q:16 * q + 16] = x
            off += 8
    assert off == row_bytes
    return out


def _uniform(codes, bits, dv, dk):
    return _decode_mixed(codes, np.full(dk // 16, bits, np.uint8), dv, dk)


def _state(rng, dv, dk):
    return (rng.standard_normal((dv, dk)) * np.exp(rng.uniform(-2, 2, (dv, 1)))).astype(np.float32)


@pytest.mark.parametrize("rounding", [RTN, SR, BDR])
@pytest.mark.parametrize("axis,G", [(0, 16), (0, 32), (1, 16), (1, 48)])
def test_mixed_head_is_blockwise_uniform(oracle, rounding, axis, G):
    """Codes and scales of a mixed head equal, block by block, those of the
    all-INT8 and all-INT4 quantizations of the same state (same counter)."""
    rng = np.random.default_rng(400 + 7 * axis + G + rounding)
    dk, dv = 128, 96
    bb = np.array([8, 8, 4, 4, 8, 8, 4, 4], np.uint8)
    c = oracle.cfg(1, 1, dk, dv, G, rounding=rounding, seed=5, layer=2, axis=axis)
    S = _state(rng, dv, dk)
    mc, ms, _ = oracle.head_quantize(c, 0, 0, bb, S, step=9)
    c8, s8, _ = oracle.head_quantize(c, 0, 0, 8, S, step=9)
    c4, s4, _ = oracle.head_quantize(c, 0, 0, 4, S, step=9)
    assert mc.size == dv * int(np.sum(2 * bb.astype(np.int64)))
    m = _decode_mixed(mc, bb, dv, dk)
    u8, u4 = _uniform(c8, 8, dv, dk), _uniform(c4, 4, dv, dk)
    col8 = np.repeat(bb == 8, 16)
    assert np.array_equal(m[:, col8], u8[:, col8])
    assert np.array_equal(m[:, ~col8], u4[:, ~col8])
    shape = oracle.scales_shape(c)
    ms, s8, s4 = ms.reshape(shape), s8.reshape(shape), s4.reshape(shape)
    if axis == 0:
        g8 = np.repeat(bb == 8, 16)[::G]
        assert np.array_equal(ms[:, g8], s8[:, g8]) and np.array_equal(ms[:, ~g8], s4[:, ~g8])
    else:
        assert np.array_equal(ms[:, col8], s8[:, col8]) and np.array_equal(ms[:, ~col8], s4[:, ~col8])
    # the dequantized state reads the same layout
    D = oracle.head_dequantize(c, bb, mc, ms)
    sc = np.repeat(ms, G, axis=1) if axis == 0 else np.repeat(ms, G, axis=0)
    assert np.array_equal(D, (m.astype(np.float32) * sc).astype(np.float32))


@pytest.mark.parametrize("mixer", [GLA, KDA])
def test_mixed_head_step_updates_the_stored_state(oracle, mixer):
    rng = np.random.default_rng(420 + mixer)
    dk, dv, G = 64, 32, 16
    bb = np.array([4, 8, 8, 4], np.uint8)
    c = oracle.cfg(1, 1, dk, dv, G, mixer=mixer, rounding=SR, seed=3)
    codes, scales, _ = oracle.head_quantize(c, 0, 0, bb, _state(rng, dv, dk), step=0)
    for t in range(1, 5):
        prev = oracle.head_dequantize(c, bb, codes, scales).astype(np.float64)
        q = rng.standard_normal(dk)
        k = rng.standard_normal(dk)
        q, k = (q / np.linalg.norm(q)).astype(np.float32), (k / np.linalg.norm(k)).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        alpha = rng.uniform(0.8, 1.0, dk).astype(np.float32)
        beta = float(np.float32(rng.uniform(0.1, 1.0))) if mixer == KDA else 0.0
        k64 = k.astype(np.float64)
        D = prev @ np.diag(alpha.astype(np.float64))
        if mixer == KDA:
            want = D @ (np.eye(dk) - beta * np.outer(k64, k64)) + beta * np.outer(v, k64)
        else:
            want = D + np.outer(v.astype(np.float64), k64)
        o, pre, _ = oracle.head_step(c, 0, 0, bb, codes, scales, q, k, v, alpha, beta, step=t,
                                     want_pre=True)
        tol = 2e-6 * max(1.0, np.abs(want).max())
        assert np.max(np.abs(pre - want)) <= tol
        assert np.max(np.abs(o - want @ q.astype(np.float64))) <= 8 * tol


def test_bits_to_slow_channels_beat_bits_to_fast_channels(oracle):
    """Prop. "decaying error" applied per channel: with the same bit budget,
    INT8 on the slowly decaying key channels and INT4 on the fast ones
    accumulates less state error than the reverse allocation."""
    rng = np.random.default_rng(440)
    dk, dv, G, T = 64, 32, 16, 96
    slow = np.repeat(np.array([True, True, False, False]), 16)
    errs = {}
    for name, bb in (("slow8", np.array([8, 8, 4, 4], np.uint8)),
                     ("fast8", np.array([4, 4, 8, 8], np.uint8))):
        e_sum = 0.0
        for rep in range(6):
            r2 = np.random.default_rng(1000 + rep)
            c = oracle.cfg(1, 1, dk, dv, G, mixer=GLA, rounding=SR, seed=rep)
            codes, scales, _ = oracle.head_quantize(c, 0, 0, bb, np.zeros((dv, dk), np.float32), 0)
            S = np.zeros((dv, dk))
            for t in range(1, T + 1):
                k = r2.standard_normal(dk)
                k = (k / np.linalg.norm(k)).astype(np.float32)
                v = r2.standard_normal(dv).astype(np.float32)
                alpha = np.where(slow, 0.999, 0.8).astype(np.float32)
                q = k
                oracle.head_step(c, 0, 0, bb, codes, scales, q, k, v, alpha, 0.0, step=t)
                S = S * alpha.astype(np.float64) + np.outer(v, k)
            e_sum += np.linalg.norm(oracle.head_dequantize(c, bb, codes, scales) - S)
        errs[name] = e_sum
    assert errs["slow8"] < 0.5 * errs["fast8"], errs


def test_batch_layout_with_block_bits(oracle):
    """Per-head block widths [H][dk/16]: head offsets and the batch entry
    points agree with the per-head ones."""
    rng = np.random.default_rng(460)
    B, H, dk, dv, G = 2, 3, 64, 16, 16
    bb = np.array([[8, 4, 4, 8], [4, 4, 4, 4], [8, 8, 8, 4]], np.uint8)
    c = oracle.cfg(B, H, dk, dv, G, mixer=GDN, rounding=SR, seed=2)
    sizes = [dv * int(np.sum(2 * bb[h].astype(np.int64))) for h in range(H)]
    assert oracle.codes_bytes(c, bb) == B * sum(sizes)
    assert oracle.head_offset(c, 1, 2, bb) == sum(sizes) + sizes[0] + sizes[1]
    S = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
    codes, scales = oracle.quantize(c, bb, S, 0)
    q = rng.standard_normal((B, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, dv)).astype(np.float32)
    alpha = rng.uniform(0.5, 1, (B, H)).astype(np.float32)
    beta = rng.uniform(0, 1, (B, H)).astype(np.float32)
    c2, s2 = codes.copy(), scales.copy()
    o = oracle.step(c, bb, c2, s2, q, k, v, alpha, beta, 1)
    for b in range(B):
        for h in range(H):
            off = oracle.head_offset(c, b, h, bb)
            hc, hs = codes[off:off + sizes[h]].copy(), scales[b, h].copy()
            oh, _, _ = oracle.head_step(c, b, h, bb[h], hc, hs, q[b, h], k[b, h], v[b, h],
                                        np.float32([alpha[b, h]]), float(beta[b, h]), step=1)
            assert np.array_equal(hc, c2[off:off + sizes[h]]) and np.array_equal(hs, s2[b, h])
            assert np.array_equal(oh, o[b, h])
