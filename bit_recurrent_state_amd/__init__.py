"""Quantized recurrent-state decode step for MI355X (gfx950).

The C ABI (include/qstate.h) is implemented by libqstate.so, built from
csrc/ with hipcc; this package is its thin Python binding."""

from .qstate import (BDR, GDN, GLA, KDA, KEY_AXIS, RTN, SCALAR, SR, VALUE_AXIS, Config, QState, qstate_bits_by_decay,  # noqa
                     qstate_create, qstate_destroy, qstate_get_step, qstate_load_fp32,
                     qstate_readout, qstate_set_step, qstate_state_bytes, qstate_step,
                     qstate_store_fp32)
