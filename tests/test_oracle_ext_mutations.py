"""Planted mistakes in the oracle's forward extras (``oracle.scan_fwd_ext``):
each mutant is the real function with one plausible error, and at least one
pin of tests/test_oracle_ext_pins.py must fail against it.  CPU only."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import test_oracle_ext_pins as pins

_real = oracle.scan_fwd_ext


def _silu(z):
    return z * expit(z)


def bias_after_softplus(s, x, dt, A, B, C, D, ids, *, dt_bias=None, dt_softplus=False, **kw):
    if dt_bias is not None and dt_softplus:
        dt = np.logaddexp(0.0, np.asarray(dt, np.float64)) + dt_bias
        return _real(s, x, dt, A, B, C, D, ids, **kw)
    return _real(s, x, dt, A, B, C, D, ids, dt_bias=dt_bias, dt_softplus=dt_softplus, **kw)


def gate_logistic_only(s, x, dt, A, B, C, D, ids, *, z=None, **kw):
    y, st, cs = _real(s, x, dt, A, B, C, D, ids, **kw)
    return (y if z is None else y * expit(z)), st, cs


def gate_skips_D(s, x, dt, A, B, C, D, ids, *, z=None, **kw):
    """D.u added after the gate (the no-conv forms, where u = x)."""
    y, st, cs = _real(s, x, dt, A, B, C, D, ids, **kw)
    if z is None or kw.get("conv_w") is not None or D is None:
        return y, st, cs
    Du = np.asarray(D)[None, :, None] * np.asarray(x)
    return (y - Du) * _silu(z) + Du, st, cs


def spans_one_long(s, x, dt, A, B, C, D, ids, *, cu_seqlens=None, **kw):
    if cu_seqlens is None:
        return _real(s, x, dt, A, B, C, D, ids, **kw)
    cu = np.asarray(cu_seqlens).copy()
    cu[1:-1] += 1
    cu = np.minimum(np.maximum.accumulate(cu), cu[-1])
    return _real(s, x, dt, A, B, C, D, ids, cu_seqlens=cu, **kw)


def rows_by_sequence(s, x, dt, A, B, C, D, ids, **kw):
    """Sequence i starts from state row i instead of ids[i]."""
    return _real(s, x, dt, A, B, C, D, np.arange(len(ids), dtype=np.int32), **kw)


def conv_state_ignored(s, x, dt, A, B, C, D, ids, *, conv_state=None, **kw):
    return _real(s, x, dt, A, B, C, D, ids, conv_state=None, **kw)


def empty_span_zero_state(s, x, dt, A, B, C, D, ids, *, cu_seqlens=None, **kw):
    y, st, cs = _real(s, x, dt, A, B, C, D, ids, cu_seqlens=cu_seqlens, **kw)
    if cu_seqlens is not None:
        st = st.copy()
        st[np.diff(np.asarray(cu_seqlens)) == 0] = 0.0
    return y, st, cs


MUTANTS = [bias_after_softplus, gate_logistic_only, gate_skips_D, spans_one_long, rows_by_sequence,
           conv_state_ignored, empty_span_zero_state]

PINS = [(pins.test_ext_equal_spans_equal_batched, dict(form="m1")),
        (pins.test_ext_equal_spans_equal_batched, dict(form="m2")),
        (pins.test_ext_split_chain_equals_unsplit, {}),
        (pins.test_ext_zero_length_sequences, {}),
        (pins.test_ext_gate_and_bias, dict(form="m1")),
        (pins.test_ext_gate_and_bias, dict(form="m2"))]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_each_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "scan_fwd_ext", mutant)
    caught = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin catches {mutant.__name__}"


def test_pins_pass_on_the_real_oracle():
    for fn, kw in PINS:
        fn(**kw)
