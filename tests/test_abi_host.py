"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point of include/qstate.h, and validates its arguments before
touching a device."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from bit_recurrent_state_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from bit_recurrent_state_amd._lib import lib
    return lib()


def _header_functions(header="qstate.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(qstate_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert len(names) >= 11
    from bit_recurrent_state_amd._lib import CEILING_EXPORTS, EXPORTS
    assert sorted(EXPORTS) == names
    ceiling = _header_functions("qstate_ceiling.h")
    assert sorted(CEILING_EXPORTS) == ceiling and len(ceiling) == 2
    for n in names + ceiling:
        assert hasattr(L, n), n


def test_ceiling_kernels_check_arguments(L):
    """Null, misaligned, odd-sized, overlapping or bad-flag calls are refused
    before any launch."""
    P = ctypes.c_void_p
    a, b = P(4096), P(4096 + (1 << 20))
    assert L.qstate_ceiling_copy(None, b, 1024, 1, None) == -1
    assert L.qstate_ceiling_copy(a, P(4096 + 8), 1024, 1, None) == -1
    assert L.qstate_ceiling_copy(a, b, 1000, 1, None) == -1
    assert L.qstate_ceiling_copy(a, b, 1024, 2, None) == -1
    assert L.qstate_ceiling_copy(a, P(4096 + 512), 1024, 0, None) == -1  # overlap
    assert L.qstate_ceiling_copy(a, b, 0, 1, None) == 0  # nothing to move
    assert L.qstate_ceiling_rmw(None, 1024, 1, 1, None) == -1
    assert L.qstate_ceiling_rmw(P(4100), 1024, 1, 1, None) == -1
    assert L.qstate_ceiling_rmw(a, 24, 1, 0, None) == -1
    assert L.qstate_ceiling_rmw(a, 0, 1, 0, None) == 0


def _cfg(**kw):
    from bit_recurrent_state_amd._lib import QStateConfig
    base = dict(batch=2, heads=3, dk=128, dv=64, group=32, mixer=0, rounding=1, fp32_state=0,
                head_bits=None, seed=1, layer=2)
    base.update(kw)
    return QStateConfig(**base)


def _bits(*b):
    arr = (ctypes.c_uint8 * len(b))(*b)
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8))


def test_state_bytes(L):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    keep, hb = _bits(4, 8, 4)
    c = _cfg(head_bits=hb)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 2 * 64 * 128 * (4 + 8 + 4) // 8
    assert sb.value == 2 * 3 * 64 * (128 // 32) * 4
    c = _cfg(fp32_state=1)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 2 * 3 * 64 * 128 * 4 and sb.value == 0
    # per-channel widths: 16 bytes per INT8 block and 8 per INT4 block of a row
    keepc = (ctypes.c_uint8 * 24)(*([8, 4, 4, 4, 8, 8, 4, 4] * 3))
    c = _cfg(channel_bits=ctypes.cast(keepc, ctypes.POINTER(ctypes.c_uint8)), group=16)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 2 * 3 * 64 * (3 * 16 + 5 * 8)
    # key-axis groups: G value rows per scale, [dv/G][dk] scales per head
    c = _cfg(head_bits=hb, group_axis=1, dk=64, dv=128, group=128)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 2 * 128 * 64 * (4 + 8 + 4) // 8
    assert sb.value == 2 * 3 * (128 // 128) * 64 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -1), (dict(heads=0), -1), (dict(dv=0), -1), (dict(mixer=4), -1),
    (dict(rounding=3), -1), (dict(group=48), -1), (dict(fp32_state=2), -1),
    (dict(dk=96, group=32), -2), (dict(dk=512, group=64), -2), (dict(heads=300), -2),
    (dict(dv=5000), -2), (dict(group=8), -2), (dict(group_axis=2), -1),
    (dict(group_axis=1, dv=48, group=32), -1), (dict(group_axis=1, dv=64, group=48), -1),
])
def test_invalid_configs_rejected(L, kw, status):
    c = _cfg(**kw)
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == status
    h = ctypes.c_void_p()
    assert L.qstate_create(ctypes.byref(c), ctypes.c_void_p(4096), ctypes.c_void_p(8192),
                           ctypes.byref(h)) == status
    assert h.value is None


def test_channel_bits_rules(L):
    """Widths 4 or 8 only; value-axis groups may not mix widths (key-axis may)."""
    def status(widths, **kw):
        arr = (ctypes.c_uint8 * 24)(*widths)
        c = _cfg(channel_bits=ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8)), **kw)
        cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
        return L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb))
    pairs = [8, 8, 4, 4, 8, 8, 4, 4] * 3
    mixed = [8, 4, 4, 8, 8, 4, 4, 8] * 3
    assert status(pairs, group=32) == 0
    assert status(mixed, group=32) == -1
    assert status(mixed, group=16) == 0
    assert status(mixed, group=32, group_axis=1) == 0
    assert status([8, 6] + [8] * 22, group=16) == -1


def test_window_rules_and_size(L):
    """Window lengths 4, 8, 16 with value-axis groups and heads of one width;
    its area follows the codes, 16-byte aligned."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    keep, hb = _bits(4, 8, 4)
    c = _cfg(head_bits=hb, window=8)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    codes = 2 * 64 * 128 * (4 + 8 + 4) // 8
    per_head = (64 * 8 + 2 * (8 * 128 + 8 * 8) + 15) // 16 * 16
    assert cb.value == (codes + 15) // 16 * 16 + 2 * 3 * per_head
    for kw, st in ((dict(window=5), -2), (dict(window=-1), -1), (dict(window=8, group_axis=1), -2),
                   (dict(window=32), -2)):
        c = _cfg(**kw)
        assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == st, kw


def test_bypass_rules(L):
    """The low-rank bypass needs a window and a finite threshold >= 0; it
    keeps the window's area."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    c = _cfg(window=8)
    assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
    pw_bytes = cb.value
    for thr in (0.0, 0.5, 3.0):
        c = _cfg(window=8, window_merge=1, lrb_threshold=thr)
        assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == 0
        assert cb.value == pw_bytes
    for kw in (dict(window=0, window_merge=1), dict(window=8, window_merge=2),
               dict(window=8, window_merge=-1), dict(window=8, window_merge=1, lrb_threshold=-0.5),
               dict(window=8, window_merge=1, lrb_threshold=float("inf")),
               dict(window=8, window_merge=1, lrb_threshold=float("nan")),
               dict(window=8, window_merge=1, fp32_state=1)):
        c = _cfg(**kw)
        assert L.qstate_state_bytes(ctypes.byref(c), ctypes.byref(cb), ctypes.byref(sb)) == -1, kw


def test_bad_head_bits_and_pointers(L):
    keep, hb = _bits(4, 6, 8)
    c = _cfg(head_bits=hb)
    h = ctypes.c_void_p()
    assert L.qstate_create(ctypes.byref(c), ctypes.c_void_p(4096), ctypes.c_void_p(8192),
                           ctypes.byref(h)) == -1
    c = _cfg()
    for codes, scales in ((0, 8192), (4096, 0), (4100, 8192), (4096, 8196)):
        assert L.qstate_create(ctypes.byref(c), ctypes.c_void_p(codes or None),
                               ctypes.c_void_p(scales or None), ctypes.byref(h)) == -1


def test_handle_lifecycle_and_argument_checks(L):
    """Create (host only), counters, and synchronous rejection of bad step
    arguments: none of these reach the device."""
    c = _cfg()
    h = ctypes.c_void_p()
    assert L.qstate_create(ctypes.byref(c), ctypes.c_void_p(4096), ctypes.c_void_p(8192),
                           ctypes.byref(h)) == 0
    step = ctypes.c_uint64()
    assert L.qstate_get_step(h, ctypes.byref(step)) == 0 and step.value == 0
    assert L.qstate_set_step(h, 41) == 0
    assert L.qstate_get_step(h, ctypes.byref(step)) == 0 and step.value == 41
    P = ctypes.c_void_p
    ok = P(1 << 20)
    # null q, misaligned k, missing beta for GDN
    assert L.qstate_step(h, None, ok, ok, ok, ok, None, None) == -1
    assert L.qstate_step(h, ok, P((1 << 20) + 4), ok, ok, ok, None, None) == -1
    assert L.qstate_step(h, ok, ok, ok, ok, None, None, None) == -1
    assert L.qstate_readout(h, ok, None, None) == -1
    assert L.qstate_load_fp32(h, P((1 << 20) + 8), None) == -1
    assert L.qstate_store_fp32(h, None, None) == -1
    assert L.qstate_get_step(h, ctypes.byref(step)) == 0 and step.value == 41  # unchanged
    assert L.qstate_destroy(h) == 0
    assert L.qstate_destroy(None) == 0
    assert L.qstate_strerror(0) == b"ok"
    assert L.qstate_strerror(-2).startswith(b"unsupported")


def test_bits_by_decay_matches_rules(L):
    from bit_recurrent_state_amd.qstate import qstate_bits_by_decay
    ret = np.array([0.95, 0.995, 0.991, 0.99, 0.90, 0.999], np.float32)
    assert qstate_bits_by_decay(ret, 0, 0.99).tolist() == [4, 8, 8, 4, 4, 8]
    ret = np.array([0.5, 0.9, 0.7, 0.9, 0.1, 0.7], np.float32)
    assert qstate_bits_by_decay(ret, 1, 0.5).tolist() == [4, 8, 8, 8, 4, 4]
    with pytest.raises(Exception):
        qstate_bits_by_decay(ret, 1, 1.5)


def test_bits_by_decay_agrees_with_reference(L, oracle):
    from bit_recurrent_state_amd.qstate import qstate_bits_by_decay
    rng = np.random.default_rng(5)
    for _ in range(100):
        ret = rng.choice([0.1, 0.5, 0.9, 0.95, 0.99, 0.999], 32).astype(np.float32)
        for mode, arg in ((0, 0.99), (1, 0.5), (1, 0.25)):
            assert np.array_equal(qstate_bits_by_decay(ret, mode, arg),
                                  oracle.bits_by_decay(ret, mode, arg))


def test_product_package_does_not_use_the_reference():
    """The product path never imports, links or loads the CPU reference."""
    pkg = os.path.join(ROOT, "bit_recurrent_state_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
