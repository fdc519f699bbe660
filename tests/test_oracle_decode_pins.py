"""Pins for the oracle's single-token decode step ("mambazip mamba1/model.rs",
forward_impl's per-token step), checked against the separately pinned
sequence scan and against exact special cases, never against the step's
formula retyped.  Each test names the mistake it would catch.  CPU only.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import ssm_inputs


def V(p, name):
    a = p.value(name)
    return None if a is None else a.astype(np.float64)


def _scan_problem(form, seed):
    if form == "m1":   # Mamba-1 with the fused conv and a carried conv state
        kw = dict(n_seqs=3, n_tokens=7, n_head=4, d_state=5, d_conv=4, conv_state_std=0.7)
    elif form == "m1k2":
        kw = dict(n_seqs=2, n_tokens=5, n_head=3, d_state=3, d_conv=2, conv_state_std=0.7)
    else:              # Mamba-2: scalar A per head, two groups, head_dim 3, no conv
        kw = dict(n_seqs=3, n_tokens=6, n_head=4, head_dim=3, d_state=4, n_group=2,
                  a_per_state=False, d_conv=0)
    return ssm_inputs.make_problem(io="f32", seed=seed, h0_std=0.5, n_state_rows=5, ids="perm",
                                   A_kind="uniform", A_range=(0.2, 2.0), **kw)


def _decode_run(p, softplus, conv_state):
    """Feed the scan problem's tokens one at a time through the decode step."""
    s = V(p, "s")
    cs = conv_state
    ys = []
    for t in range(p.n_tokens):
        y, s, cs = oracle.state_update(s, V(p, "x")[:, t], V(p, "dt")[:, t], V(p, "A"),
                                       V(p, "B")[:, t], V(p, "C")[:, t], V(p, "D"), p.ids,
                                       conv_w=V(p, "conv_w") if p.d_conv else None,
                                       conv_state=cs, dt_softplus=softplus)
        ys.append(y)
    return np.stack(ys, axis=1), s, cs


# --------------------------------------------------------------------------
# L decode steps from the gathered state rows equal one L-token scan: the
# y of every token, the final state (scan row i against decode row ids[i])
# and the conv state.  Catches: a wrong tap order or window in the ring, a
# missing or misplaced ring shift, the state updated after y, a dropped D,
# a wrong group map, a state written to the sequence row instead of its id.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form,softplus", [("m1", False), ("m1k2", True), ("m2", False), ("m2", True)])
def test_decode_steps_equal_scan(form, softplus):
    p = _scan_problem(form, 41)
    p.dt_softplus = softplus
    cs0 = V(p, "conv_state") if p.d_conv else None
    y_scan, st_scan, cso = oracle.scan_fwd(V(p, "s"), V(p, "x"), V(p, "dt"), V(p, "A"), V(p, "B"),
                                           V(p, "C"), V(p, "D"), p.ids,
                                           conv_w=V(p, "conv_w") if p.d_conv else None,
                                           conv_state=cs0, dt_softplus=softplus)
    y_dec, s_dec, cs_dec = _decode_run(p, softplus, cs0)
    np.testing.assert_allclose(y_dec, y_scan, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s_dec[p.ids], st_scan, rtol=1e-12, atol=1e-13)
    if p.d_conv:
        np.testing.assert_allclose(cs_dec[p.ids], cso, rtol=0, atol=0)


# --------------------------------------------------------------------------
# dt = 0 (no softplus): a = 1 and b = 0, so every state row is returned bit
# for bit and y = C.h0 + D.u.  Rows no id names are never touched.
# Catches: a decay that is not exp(0) = 1, an input term without dt, a write
# to the wrong row, a write to rows outside ids.
# --------------------------------------------------------------------------
def test_decode_dt_zero_and_untouched_rows():
    p = _scan_problem("m2", 43)
    s0 = V(p, "s")
    dt0 = np.zeros((p.n_seqs, p.n_head))
    y, s1, _ = oracle.state_update(s0, V(p, "x")[:, 0], dt0, V(p, "A"), V(p, "B")[:, 0],
                                   V(p, "C")[:, 0], V(p, "D"), p.ids)
    assert np.array_equal(s1, s0)
    B0, C0, x0 = V(p, "B")[:, 0], V(p, "C")[:, 0], V(p, "x")[:, 0]
    grp = oracle.group_of_head(p.n_head, p.n_group)
    want = np.einsum("ihpn,ihn->ihp", s0[p.ids], C0[:, grp]) + V(p, "D")[None, :, None] * x0
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-14)
    # a real step changes exactly the rows ids names
    _, s2, _ = oracle.state_update(s0, x0, V(p, "dt")[:, 0], V(p, "A"), B0, C0, V(p, "D"), p.ids)
    untouched = np.setdiff1d(np.arange(s0.shape[0]), p.ids)
    assert np.array_equal(s2[untouched], s0[untouched])
    assert not np.array_equal(s2[p.ids], s0[p.ids])


# --------------------------------------------------------------------------
# The conv ring holds the last K-1 inputs, oldest first, exactly: after K-1
# steps with inputs v1..v_{K-1} the state rows are those inputs, whatever
# they held before.  Catches: a ring that shifts the wrong way, drops the
# newest input or keeps the oldest.
# --------------------------------------------------------------------------
def test_decode_conv_ring_keeps_last_inputs():
    p = _scan_problem("m1", 47)
    K = p.d_conv
    cs = V(p, "conv_state")
    s = V(p, "s")
    xs = V(p, "x")
    for t in range(K - 1):
        _, s, cs = oracle.state_update(s, xs[:, t], V(p, "dt")[:, t], V(p, "A"), V(p, "B")[:, t],
                                       V(p, "C")[:, t], V(p, "D"), p.ids, conv_w=V(p, "conv_w"),
                                       conv_state=cs)
    want = np.moveaxis(xs[:, :K - 1, :, 0], 1, 2)  # [S][H][K-1], oldest first
    assert np.array_equal(cs[p.ids], want)


# --------------------------------------------------------------------------
# The z gate multiplies y by SiLU(z) = z * logistic(z) (scipy's expit), and
# the dt bias is added before softplus: a step with (dt, bias) equals a step
# with dt + bias and no bias, and with softplus on it equals a step whose dt
# is softplus(dt + bias) (numpy's logaddexp) with softplus off.
# Catches: a gate of logistic(z) alone, the gate applied to the state, the
# bias added after softplus or with the wrong sign.
# --------------------------------------------------------------------------
def test_decode_gate_and_dt_bias():
    p = _scan_problem("m2", 53)
    rng = np.random.default_rng(5)
    z = rng.normal(size=(p.n_seqs, p.n_head, p.head_dim))
    bias = rng.uniform(-1, 1, p.n_head)
    args = (V(p, "s"), V(p, "x")[:, 0], V(p, "dt")[:, 0], V(p, "A"), V(p, "B")[:, 0],
            V(p, "C")[:, 0], V(p, "D"), p.ids)
    y_plain, s_plain, _ = oracle.state_update(*args)
    y_gate, s_gate, _ = oracle.state_update(*args, z=z)
    np.testing.assert_allclose(y_gate, y_plain * z * expit(z), rtol=1e-13, atol=1e-15)
    assert np.array_equal(s_gate, s_plain)

    dt0 = V(p, "dt")[:, 0]
    a2 = list(args)
    a2[2] = dt0 + bias[None, :]
    y_b, s_b, _ = oracle.state_update(*args, dt_bias=bias)
    y_sum, s_sum, _ = oracle.state_update(*a2)
    np.testing.assert_allclose(y_b, y_sum, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s_b, s_sum, rtol=1e-14, atol=1e-15)

    a3 = list(args)
    a3[2] = np.logaddexp(0.0, dt0 + bias[None, :])
    y_sp, s_sp, _ = oracle.state_update(*args, dt_bias=bias, dt_softplus=True)
    y_pre, s_pre, _ = oracle.state_update(*a3)
    np.testing.assert_allclose(y_sp, y_pre, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s_sp, s_pre, rtol=1e-12, atol=1e-14)
