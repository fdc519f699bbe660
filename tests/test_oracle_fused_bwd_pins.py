"""Pins for the oracle's backward through the fused conv + SiLU (the scan
consuming u = SiLU(causal depthwise conv of x), conv taps in the order of
the ggml ssm_conv test on "ggmlR tests/testthat/test-ssm-rwkv.R", the last
tap on the newest input, with d_conv-1 conv-state inputs before the first
token):

- central differences in float64 of the fused forward, for every input
  including the conv weights and the gathered conv-state rows (repeated ids
  accumulate into one row);
- the adjoint identity <dout, J v> = <J^T dout, v>, J v by the complex step
  of an independent numpy forward;
- with a unit last tap the conv passes x through, so nothing reaches the
  conv state and d_x is the unfused gradient of u times SiLU's derivative.
CPU only.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs

NAMES = ("s", "x", "dt", "A", "B", "C", "D", "conv_w", "conv_state")


def _problem(seed, K, L, **kw):
    base = dict(n_seqs=3, n_tokens=L, n_head=3, d_state=4, d_conv=K, io="f32", seed=seed,
                h0_std=0.7, A_kind="uniform", A_range=(0.2, 1.0), n_state_rows=3,
                ids=np.array([2, 0, 2], np.int32), with_dout=True, dstate_std=1.0,
                conv_state_std=0.8)
    base.update(kw)
    return ssm_inputs.make_problem(**base)


def _vals(p):
    return {k: p.value(k).astype(np.float64).copy() for k in NAMES}


def _loss(p, v, w_y, w_s):
    y, st, _ = oracle.scan_fwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids,
                               conv_w=v["conv_w"], conv_state=v["conv_state"],
                               dt_softplus=p.dt_softplus, n_threads=1)
    return float(np.sum(y * w_y) + np.sum(st * w_s))


def _grads(p, v, w_y, w_s):
    return oracle.scan_bwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids, w_y, w_s,
                           conv_w=v["conv_w"], conv_state=v["conv_state"],
                           dt_softplus=p.dt_softplus, n_threads=2)


@pytest.mark.parametrize("K,L,softplus", [(4, 5, False), (3, 6, True), (2, 4, False), (4, 2, False)])
def test_fused_backward_matches_central_differences(K, L, softplus):
    """Catches a wrong tap in the conv adjoint, a missing SiLU derivative, a
    conv-state gradient sent to the wrong row or not accumulated over
    repeated ids, and any wrong term of the scan's own gradients."""
    p = _problem(11 + K + L, K, L)
    p.dt_softplus = softplus
    v = _vals(p)
    if softplus:
        v["dt"] = v["dt"] * 6.0 - 2.0
    w_y, w_s = p.value("dy").astype(np.float64), p.value("dstate").astype(np.float64)
    g = _grads(p, v, w_y, w_s)
    eps = 1e-6
    for name in NAMES:
        base = v[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            old = base[idx]
            base[idx] = old + eps
            lp = _loss(p, v, w_y, w_s)
            base[idx] = old - eps
            lm = _loss(p, v, w_y, w_s)
            base[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(g["d_" + name], num, rtol=1e-6, atol=1e-7 * scale, err_msg=name)


def _np_fused_forward(v, ids, K):
    """Independent forward: conv as the valid correlation of [conv state | x]
    with each channel's taps (written out: numpy's correlate conjugates a
    complex second operand), SiLU, then the decays' running product."""
    x, dt, A, B, C, D, s, w, cs = (v[k] for k in ("x", "dt", "A", "B", "C", "D", "s", "conv_w",
                                                  "conv_state"))
    S, L, H, _ = x.shape
    u = np.zeros((S, L, H), dtype=complex)
    for i in range(S):
        for h in range(H):
            row = np.concatenate([cs[ids[i], h], x[i, :, h, 0]])
            u[i, :, h] = sum(w[h, j] * row[j:j + L] for j in range(K))
    u = u / (1.0 + np.exp(-u))
    h_st = s[ids][:, :, 0, :].astype(complex)
    ys = []
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None])
        h_st = a * h_st + dt[:, t, :, None] * B[:, t, 0][:, None, :] * u[:, t, :, None]
        ys.append(np.einsum("shn,sn->sh", h_st, C[:, t, 0]) + D[None] * u[:, t])
    return np.stack(ys, axis=1)[..., None], h_st[:, :, None, :]


def test_fused_adjoint_identity_with_complex_step():
    p = _problem(61, 4, 7)
    v = _vals(p)
    rng = np.random.default_rng(8)
    direction = {k: rng.standard_normal(v[k].shape) for k in NAMES}
    step = 1e-30
    vc = {k: v[k] + 1j * step * direction[k] for k in NAMES}
    yc, sc = _np_fused_forward(vc, p.ids, 4)
    w_y, w_s = p.value("dy").astype(np.float64), p.value("dstate").astype(np.float64)
    jvp = (np.sum(w_y * yc.imag) + np.sum(w_s * sc.imag)) / step
    g = _grads(p, v, w_y, w_s)
    vjp = sum(np.sum(g["d_" + k] * direction[k]) for k in NAMES)
    assert abs(jvp - vjp) <= 1e-11 * max(1.0, abs(jvp)), (jvp, vjp)
    y, st, _ = oracle.problem_fwd(p)
    yr, sr = _np_fused_forward(v, p.ids, 4)
    np.testing.assert_allclose(y, yr.real, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, sr.real, rtol=1e-12, atol=1e-13)


def test_unit_last_tap_passes_x_through():
    """w = (0, .., 0, 1): u_t = SiLU(x_t).  The conv state meets only zero
    taps (its gradient is zero) and d_x = (unfused d_u at u = SiLU(x)) *
    SiLU'(x), with SiLU'(c) = sigma(c) (1 + c (1 - sigma(c)))."""
    p = _problem(71, 4, 6)
    v = _vals(p)
    v["conv_w"][:] = 0.0
    v["conv_w"][:, -1] = 1.0
    w_y, w_s = p.value("dy").astype(np.float64), p.value("dstate").astype(np.float64)
    g = _grads(p, v, w_y, w_s)
    assert not np.any(g["d_conv_state"])
    x = v["x"]
    sg = 1.0 / (1.0 + np.exp(-x))
    u = x * sg
    g0 = oracle.scan_bwd(v["s"], u, v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids, w_y, w_s)
    np.testing.assert_allclose(g["d_x"], g0["d_x"] * sg * (1.0 + x * (1.0 - sg)), rtol=1e-12,
                               atol=1e-14)
    for k in ("d_s", "d_dt", "d_A", "d_B", "d_C", "d_D"):
        np.testing.assert_allclose(g[k], g0[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_zero_upstream_gives_zero_fused_gradients():
    p = _problem(81, 3, 5)
    v = _vals(p)
    g = _grads(p, v, np.zeros_like(p.value("dy"), dtype=np.float64),
               np.zeros_like(p.value("dstate"), dtype=np.float64))
    for k, arr in g.items():
        assert not np.any(arr), k
