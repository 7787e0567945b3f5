"""Host-side checks of bench.py's measurement bookkeeping (no GPU needed):
the algorithmic bytes of a step against figures counted by hand from the
state layout, the per-kernel rocprofv3 records (HBM traffic, VALU
instructions) tied to the kernel source they were taken on, and the
one-GPU guard."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def Q():
    from bit_recurrent_state_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from bit_recurrent_state_amd import qstate
    return qstate


def test_algorithmic_bytes_headline(Q):
    """Gated DeltaNet, B=256, H=32, dk=dv=128, group 32: one head per batch row
    (alpha_h > 0.99) is INT8, the other 31 are INT4.  Per head the codes
    (dv*dk*n/8) and scales (dv*dk/G*4) are read and written once; q, k, v, o
    are 4*(2*128 + 2*128) bytes; alpha and beta 4 bytes each."""
    import bench
    import workloads as W
    w = W.WORKLOADS[2]
    bb = bench.block_bits(w, Q)
    assert sorted(set(bb.ravel().tolist())) == [4, 8]
    assert int((bb[:, 0] == 8).sum()) == 1
    int4_head = 2 * (128 * 128 // 2 + 128 * 4 * 4)  # 20480
    int8_head = 2 * (128 * 128 + 128 * 4 * 4)       # 36864
    io, gates = 4 * (2 * 128 + 2 * 128), 8
    per_b = 31 * int4_head + int8_head + 32 * (io + gates)
    assert bench.algorithmic_bytes(w, bb) == 256 * per_b == 188_809_216


def test_algorithmic_bytes_gla(Q):
    """GLA, B=256, H=16, dk=dv=128, INT8, group 64: alpha is one float per key
    channel, no beta."""
    import bench
    import workloads as W
    w = W.WORKLOADS[3]
    bb = bench.block_bits(w, Q)
    assert set(bb.ravel().tolist()) == {8}
    head = 2 * (128 * 128 + 128 * 2 * 4) + 4 * (2 * 128 + 2 * 128) + 4 * 128
    assert bench.algorithmic_bytes(w, bb) == 256 * 16 * head == 153_092_096


def test_fp32_state_bytes():
    import bench
    import workloads as W
    w = W.WORKLOADS[2]
    head = 2 * 128 * 128 * 4 + 4 * (2 * 128 + 2 * 128) + 8
    assert bench.fp32_bytes(w) == 256 * 32 * head


def test_profile_records_follow_the_kernel_source(monkeypatch):
    """The stored traffic and VALU counts are reported only while the kernel
    source hash matches the one they were measured on."""
    import bench
    import workloads as W
    rec = json.load(open(bench.TRAFFIC_FILE))
    w = W.WORKLOADS[2]
    entry = rec["workloads"].get(bench.traffic_key(w))
    assert entry is not None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w_: entry["kernel_source_sha256_16"])
    assert bench.measured_traffic(w) == entry["hbm_bytes_per_launch"]
    assert bench.measured_valu(w) == entry.get("valu_wave_insts_per_launch")
    assert bench.measured_clock(w) == entry.get("shader_clock_ghz")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w_: "0" * 16)
    assert bench.measured_traffic(w) is None
    assert bench.measured_valu(w) is None
    assert bench.measured_clock(w) is None


def test_stored_records_are_calibrated():
    """Each stored record scales FETCH_SIZE by 2 and WRITE_SIZE by 1, the
    factors the library's 2 GiB in-place read-modify-write kernel gives on
    gfx950."""
    import bench
    rec = json.load(open(bench.TRAFFIC_FILE))
    for key, e in rec["workloads"].items():
        assert len(e["kernel_source_sha256_16"]) == 16, key
        assert e["hbm_bytes_per_launch"] > 0, key
        assert e["fetch_scale"] == pytest.approx(2.0, rel=1e-3), key
        assert e["write_scale"] == pytest.approx(1.0, rel=1e-3), key


def test_traffic_close_to_algorithmic_bytes(Q):
    """Measured HBM bytes within 10 % above the algorithmic ones: every state
    byte read once and written once, no re-reads."""
    import bench
    import workloads as W
    rec = json.load(open(bench.TRAFFIC_FILE))["workloads"]
    for wid in (2, 3):
        w = W.WORKLOADS[wid]
        e = rec[bench.traffic_key(w)]
        alg = bench.algorithmic_bytes(w, bench.block_bits(w, Q))
        assert 1.0 <= e["hbm_bytes_per_launch"] / alg < 1.10, (wid, e["hbm_bytes_per_launch"], alg)


def test_unit_hash_follows_its_includes(tmp_path, monkeypatch):
    """A kernel unit's hash covers the headers it includes and no others."""
    from bit_recurrent_state_amd import build
    src = tmp_path / "csrc"
    inc = tmp_path / "include"
    src.mkdir()
    inc.mkdir()
    (src / "a.hip").write_text('#include "h1.h"\n')
    (src / "h1.h").write_text('#include "h2.h"\n')
    (src / "h2.h").write_text("int x;\n")
    (src / "other.h").write_text("int y;\n")
    monkeypatch.setattr(build, "CSRC", str(src))
    monkeypatch.setattr(build, "ROOT", str(tmp_path))
    h0 = build.unit_hash("a.hip")
    (src / "other.h").write_text("int z;\n")
    assert build.unit_hash("a.hip") == h0
    (src / "h2.h").write_text("int w;\n")
    assert build.unit_hash("a.hip") != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_algorithmic_bytes_layer_stack(Q):
    """Mamba2-style stack: 24 layers, each B=512, H=32, dv=64 (head dim),
    dk=128 (state dim), group 64, half the heads INT8 (slowest decay of that
    layer) and half INT4; scalar decay: one alpha and one dt per head."""
    import bench
    import workloads as W
    w = W.WORKLOADS[4]
    assert w.layers == 24
    int8_head = 2 * (64 * 128 + 64 * 2 * 4)
    int4_head = 2 * (64 * 128 // 2 + 64 * 2 * 4)
    io, gates = 4 * (2 * 128 + 2 * 64), 8
    per_layer = 512 * (16 * int8_head + 16 * int4_head + 32 * (io + gates))
    for layer in (0, 7, 23):
        hb1 = Q.qstate_bits_by_decay(W.head_retention(w, 0, layer), 1, 0.5)
        assert int((hb1 == 8).sum()) == 16
        hb = np.repeat(hb1[:, None], w.dk // 16, axis=1).astype(np.uint8)
        assert bench.algorithmic_bytes(w, hb) == per_layer
    assert 24 * per_layer == 5_841_616_896


def test_cpu_baseline_reports_every_core_and_one(monkeypatch):
    """The reference timed on one thread and on every core of the affinity
    mask, with the CPU model; the sample runs briefly here."""
    import bench
    import workloads as W
    w = W.WORKLOADS[2]
    hb = np.repeat(np.array([4] * 31 + [8], np.uint8)[:, None], 8, axis=1)
    r = bench.cpu_baseline(w, hb, 0.3, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s"
    assert r["cores"] == bench.host_cores() >= 1
    assert r["single_thread"]["cores"] == 1
    assert r["value"] > 0 and r["single_thread"]["value"] > 0
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]


def test_profile_records_are_per_shape_and_width_mix():
    """A run with another batch or width policy never picks up the record of
    the workload's own shape and widths."""
    import bench
    import workloads as W
    w = W.WORKLOADS[2]
    keys = {bench.traffic_key(x) for x in (w, w.scaled(B=8), w.scaled(bits_policy="int8"),
                                           w.scaled(rounding=W.RTN), w.scaled(axis=1),
                                           w.scaled(window=8))}
    assert len(keys) == 6
    assert bench.traffic_key(w) == "gdn_b256_h32_d128_int4mix_g32_sr|SR|value-axis"
