"""GPU parity over the workloads' whole step counts (see tests/horizon.py).

* Full batch, every head, every step: the B=64 Gated DeltaNet INT8 SR
  workload for its 256 steps.
* Full batch, the bench's launch size: every head at the import and step 1,
  a seeded sample of heads (every head index, the first and last head) at
  every step through T = 1024 (B=256 INT4/INT8 mix), 512 (GLA, RTN and SR)
  and 256 (Mamba2-style, all 24 layer keys).
* Reduced batch (heads are independent; the same per-head workload), every
  head at every step through the same T, also with bounded directional
  rounding on the Gated DeltaNet and GLA workloads, with key-axis scale
  groups, and with per-channel widths.
Set QSTATE_PARITY_EVERY_HEAD=1 to track every head of the full batch through
T as well (minutes of host time).  Set QSTATE_PARITY_REPORT=<file> to append
one JSON line per run."""

import json
import os

import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

import workloads as W  # noqa: E402

if gpu_available():
    from horizon import Horizon, sample_heads
    from parity import log

EVERY = os.environ.get("QSTATE_PARITY_EVERY_HEAD") == "1"


def _run(w, steps, rounding=None, layer=0, tracked=None, every=None, tag=""):
    hz = Horizon(w, rounding, 0, layer, tracked, every)
    log(f"[case] horizon {tag} {w.name} B={w.B} H={w.H} dk={w.dk} dv={w.dv} G={w.G} "
        f"rounding={hz.rounding} layer={layer} steps={steps} tracked={len(hz.tracked)} "
        f"every-head-at-0-1={len(hz.every)} threads={hz.threads}")
    rep = hz.run(steps)
    line = {"case": tag, "workload": w.name, "B": w.B, "rounding": rep.rounding, "layer": layer,
            "steps": rep.steps, "heads_tracked": rep.heads_tracked,
            "heads_at_import_and_step1": rep.heads_every, "head_steps": rep.head_steps,
            "elements": rep.elements, "exempt": rep.exempt, "max_o_err": rep.max_o_err,
            "free_running": rep.free_running, "seconds": round(rep.seconds, 1)}
    log("[done] " + json.dumps(line))
    out = os.environ.get("QSTATE_PARITY_REPORT")
    if out:
        with open(out, "a") as f:
            f.write(json.dumps(line) + "\n")
    return rep


def test_config1_every_head_every_step():
    w = W.WORKLOADS[1]
    rep = _run(w, w.steps, tag="full-every")
    assert rep.head_steps == w.B * w.H * w.steps


def test_config2_full_size_sampled_heads_to_T():
    w = W.WORKLOADS[2]
    rep = _run(w, w.steps, tracked=sample_heads(w, 256, 2), every="all", tag="full-sampled")
    assert rep.heads_tracked >= 256 and rep.heads_every == w.B * w.H


@pytest.mark.parametrize("rounding", [W.RTN, W.SR])
def test_config3_full_size_sampled_heads_to_T(rounding):
    w = W.WORKLOADS[3]
    rep = _run(w, w.steps, rounding, tracked=sample_heads(w, 128, 3), every="all",
               tag="full-sampled")
    assert rep.heads_tracked >= 128


@pytest.mark.parametrize("first", [0, 6, 12, 18])
def test_config4_full_size_layers_to_T(first):
    """Six of the 24 independent layers (layer keys first..first+5) per test:
    every head of the first of them at the import and step 1, 32 sampled heads
    of each at every step through T."""
    w = W.WORKLOADS[4]
    for layer in range(first, first + 6):
        _run(w, w.steps, layer=layer, tracked=sample_heads(w, 32, 40 + layer),
             every="all" if layer == first else None, tag="full-sampled")


@pytest.mark.parametrize("wid,B,rounding", [(2, 8, None), (3, 8, W.RTN), (3, 8, W.SR),
                                            (5, 8, None), (2, 8, W.BDR), (3, 8, W.BDR)])
def test_every_head_every_step_reduced_batch(wid, B, rounding):
    w = W.WORKLOADS[wid].scaled(B=B)
    rep = _run(w, w.steps, rounding, tag=f"B{B}-every")
    assert rep.head_steps == w.B * w.H * w.steps


@pytest.mark.parametrize("wid,B,rounding", [(3, 8, W.RTN), (3, 8, W.SR), (2, 8, None),
                                            (5, 8, None), (6, 8, None)])
def test_key_axis_every_head_every_step_reduced_batch(wid, B, rounding):
    """Key-axis scale groups (the block-prefetching kernels and the plain
    one) over the workloads' whole step counts, every head."""
    w = W.WORKLOADS[wid].scaled(B=B, axis=1)
    rep = _run(w, w.steps, rounding, tag=f"B{B}-every-keyaxis")
    assert rep.head_steps == w.B * w.H * w.steps


def test_channel_bits_every_head_every_step_reduced_batch():
    """Per-channel widths (lanes of both widths in every wave) over the
    workload's whole step count, every head."""
    w = W.WORKLOADS[6].scaled(B=8)
    rep = _run(w, w.steps, tag="B8-every")
    assert rep.head_steps == w.B * w.H * w.steps


def test_config4_every_layer_every_head_reduced_batch():
    w = W.WORKLOADS[4].scaled(B=4)
    for layer in range(24):
        _run(w, w.steps, layer=layer, tag="B4-every")


@pytest.mark.skipif(not EVERY, reason="set QSTATE_PARITY_EVERY_HEAD=1 (minutes of host time)")
@pytest.mark.parametrize("wid,rounding", [(2, None), (2, W.BDR), (3, W.RTN), (3, W.SR)])
def test_full_size_every_head_to_T(wid, rounding):
    w = W.WORKLOADS[wid]
    rep = _run(w, w.steps, rounding, tag="full-every")
    assert rep.head_steps == w.B * w.H * w.steps


@pytest.mark.skipif(not EVERY, reason="set QSTATE_PARITY_EVERY_HEAD=1 (minutes of host time)")
def test_config4_full_size_every_head_one_layer():
    w = W.WORKLOADS[4]
    _run(w, w.steps, layer=23, tag="full-every")
