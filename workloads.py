"""Seeded synthetic decode workloads for the quantized recurrent-state step.

This module only draws inputs: shapes, seeds and value distributions.  It
holds none of the method's arithmetic (no update, no quantizer, no random
bits for rounding), and both the CPU reference and the HIP path consume the
exact arrays it returns.

Input recipe (per batch row b, head h, input step t):
  q, k ~ N(0, 1)^dk, each L2-normalised per head (unit keys, as the delta
         rule's contraction assumes);
  v    ~ N(0, 1)^dv;
  beta  = sigmoid(N(0, 1));
  alpha = exp(-softplus(N(-4, 1))).
Overrides per workload are listed on each entry of WORKLOADS.  Every draw is
a PCG64 stream keyed by (seed, workload id, tensor id, step[, layer]), so any
step can be regenerated alone.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

GDN, GLA, SCALAR, KDA = 0, 1, 2, 3
RTN, SR, BDR = 0, 1, 2

# tensor ids for the seed sequence
_Q, _K, _V, _BETA, _ALPHA, _HEAD_ALPHA, _HEAD_A, _DT, _CHAN_MU = range(9)


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, recurrence, storage and input recipe."""

    wid: int
    name: str
    mixer: int
    B: int
    H: int
    dk: int
    dv: int
    G: int
    steps: int
    warmup: int          # FP32 steps before the state is quantized
    rounding: int
    bits_policy: str     # "int8" | "alpha_gt_0.99" | "rank_half" | "channel_half"
    layers: int = 1
    axis: int = 0        # scale groups: 0 value axis (G key columns), 1 key axis (G value rows)
    window: int = 0      # pair buffer length W (0: none)
    window_merge: int = 0  # 0 pure-write window, 1 low-rank bypass (merge every W steps)
    lrb_threshold: float = 0.5  # low-rank bypass: merge threshold in group scales

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Single Gated-DeltaNet layer, INT8, RTN, state starts at zero.
    0: Workload(0, "gdn_b1_h4_d64_int8_g64_rtn", GDN, 1, 4, 64, 64, 64, 64, 0, RTN, "int8"),
    # Gated-DeltaNet, INT8, group 32, stochastic rounding, 32 FP32 warm-up steps.
    1: Workload(1, "gdn_b64_h16_d128_int8_g32_sr", GDN, 64, 16, 128, 128, 32, 256, 32, SR,
                "int8"),
    # Gated-DeltaNet, INT4 (INT8 for heads with alpha > 0.99), group 32, SR;
    # alpha per head ~ U(0.90, 0.999), constant over b and t.
    2: Workload(2, "gdn_b256_h32_d128_int4mix_g32_sr", GDN, 256, 32, 128, 128, 32, 1024, 32, SR,
                "alpha_gt_0.99"),
    # GLA diagonal decay alpha_j = sigmoid(N(3,1))^(1/16), INT8, group 64 (RTN and SR runs).
    3: Workload(3, "gla_b256_h16_d128_int8_g64", GLA, 256, 16, 128, 128, 64, 512, 32, RTN, "int8"),
    # Mamba2-style scalar decay, 24 independent layers, dv=64 (head dim), dk=128 (state
    # dim); alpha = exp(-softplus(a_h) * dt), a_h ~ N(-3,1) per (layer, h),
    # dt ~ U(0.001, 0.1) per (layer, b, h, t); write weight dt; half the heads
    # (slowest decay) INT8, the rest INT4; group 64; SR.
    4: Workload(4, "mamba2_24x_b512_h32_p64_n128_int8int4_g64_sr", SCALAR, 512, 32, 128, 64, 64,
                256, 32, SR, "rank_half", layers=24),
    # KDA (per-key-channel decay with delta correction) at the GLA shape: alpha_j as GLA's,
    # beta as Gated DeltaNet's; INT8, group 64, SR.
    5: Workload(5, "kda_b256_h16_d128_int8_g64_sr", KDA, 256, 16, 128, 128, 64, 512, 32, SR, "int8"),
    # GLA with a persistent decay rate per key channel: alpha_j = sigmoid(mu_hj + N(0, 0.5^2))
    # ^(1/16), mu_hj ~ N(3, 1) sorted descending inside each head (channels ordered by decay);
    # per head the slower half of the 32-channel groups INT8, the rest INT4; SR.
    6: Workload(6, "gla_b256_h16_d128_chmix_g32_sr", GLA, 256, 16, 128, 128, 32, 512, 32, SR,
                "channel_half"),
}


def _rng(seed: int, wid: int, tensor: int, *more: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor, *more])))


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _unit(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


def head_retention(w: Workload, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Per-head decay statistic (larger = slower decay) that sets the bit widths.

    alpha_gt_0.99: alpha_h itself; rank_half: exp(-softplus(a_h)); int8: ones."""
    if w.bits_policy == "alpha_gt_0.99":
        return head_alpha(w, seed)
    if w.bits_policy == "rank_half":
        return np.exp(-_softplus(head_a(w, seed, layer))).astype(np.float32)
    return np.ones(w.H, np.float32)


def channel_mu(w: Workload, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Persistent per-(head, key channel) decay logit mu_hj ~ N(3, 1), sorted
    descending inside each head ("channel_half" policy)."""
    mu = _rng(seed, w.wid, _CHAN_MU, layer).standard_normal((w.H, w.dk)) + 3.0
    return -np.sort(-mu, axis=1)


def channel_retention(w: Workload, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Per-(head, key channel) decay statistic sigmoid(mu_hj)^(1/16), float32 [H][dk]."""
    mu = channel_mu(w, seed, layer)
    return ((1.0 / (1.0 + np.exp(-mu))) ** (1.0 / 16.0)).astype(np.float32)


def group_retention(w: Workload, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Mean channel retention of each value-axis group of G key channels, [H][dk/G]."""
    r = channel_retention(w, seed, layer).astype(np.float64)
    return r.reshape(w.H, w.dk // w.G, w.G).mean(axis=2).astype(np.float32)


def head_alpha(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-head constant alpha_h ~ U(0.90, 0.999) (alpha_gt_0.99 policy)."""
    return _rng(seed, w.wid, _HEAD_ALPHA).uniform(0.90, 0.999, w.H).astype(np.float32)


def head_a(w: Workload, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Per-(layer, head) Mamba2 decay parameter a_h ~ N(-3, 1)."""
    return (_rng(seed, w.wid, _HEAD_A, layer).standard_normal(w.H) - 3.0).astype(np.float32)


def step_inputs(w: Workload, t: int, seed: int = 0, layer: int = 0):
    """Inputs of input step t: (q, k, v, alpha, beta), float32, library layout.

    q, k [B][H][dk]; v [B][H][dv]; alpha [B][H] or [B][H][dk] (GLA, KDA);
    beta [B][H] (GDN and KDA beta, scalar-decay dt) or None (GLA)."""
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    q = _unit(_normal(_rng(seed, w.wid, _Q, t, layer), (B, H, dk)))
    k = _unit(_normal(_rng(seed, w.wid, _K, t, layer), (B, H, dk)))
    v = _normal(_rng(seed, w.wid, _V, t, layer), (B, H, dv))
    if w.mixer in (GLA, KDA):
        z = _normal(_rng(seed, w.wid, _ALPHA, t, layer), (B, H, dk)).astype(np.float64)
        if w.bits_policy == "channel_half":
            z = channel_mu(w, seed, layer)[None] + 0.5 * z
        else:
            z = z + 3.0
        alpha = ((1.0 / (1.0 + np.exp(-z))) ** (1.0 / 16.0)).astype(np.float32)
        if w.mixer == GLA:
            return q, k, v, alpha, None
        zb = _normal(_rng(seed, w.wid, _BETA, t, layer), (B, H)).astype(np.float64)
        return q, k, v, alpha, (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    if w.mixer == SCALAR:
        dt = _rng(seed, w.wid, _DT, t, layer).uniform(0.001, 0.1, (B, H))
        a = head_a(w, seed, layer).astype(np.float64)
        alpha = np.exp(-_softplus(a)[None, :] * dt).astype(np.float32)
        return q, k, v, alpha, dt.astype(np.float32)
    zb = _normal(_rng(seed, w.wid, _BETA, t, layer), (B, H)).astype(np.float64)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    if w.bits_policy == "alpha_gt_0.99":
        alpha = np.broadcast_to(head_alpha(w, seed)[None, :], (B, H)).astype(np.float32)
    else:
        za = _normal(_rng(seed, w.wid, _ALPHA, t, layer), (B, H)).astype(np.float64) - 4.0
        alpha = np.exp(-_softplus(za)).astype(np.float32)
    return q, k, v, alpha, beta


def head_slice(arr, b: int, h: int):
    """The (b, h) slice of a [B][H][...] input (scalar for [B][H] arrays)."""
    if arr is None:
        return None
    return arr[b, h]
