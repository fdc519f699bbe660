"""Pins for the oracle's reverse-time backward.

- central differences in float64 of the forward (the pages' own check:
  "ggmlR test-ssm-rwkv.R" scores <whole packed result, w>, and
  "kizzasi-model backprop_ssm.rs" test_ssm_backward_finite_diff);
- the adjoint identity <dout, J v> = <J^T dout, v>, with J v taken by the
  complex-step derivative of an independent numpy forward (exact to
  rounding, no cancellation);
- zero upstream gradient gives zero gradients ("lattice-inference
  gdn_backward.rs", zero_grad_output_yields_zero_input_grad);
- the time-invariant special case against the backward equations of
  "kizzasi-model backprop_ssm.rs" (ssm_backward).
CPU only.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs

NAMES = ("s", "x", "dt", "A", "B", "C", "D")


def _problem(form, seed, **kw):
    base = dict(n_seqs=2, n_tokens=5, n_head=3, d_state=4, d_conv=0, io="f32", seed=seed,
                h0_std=0.7, A_kind="uniform", A_range=(0.2, 1.0), n_state_rows=3,
                ids=np.array([2, 0], np.int32), with_dout=True, dstate_std=1.0)
    if form == "m2":
        # the ggmlR FD shapes: d_state 3, head_dim 2, n_head 2, 3 tokens, 1 sequence
        base.update(n_seqs=1, n_tokens=3, n_head=2, head_dim=2, d_state=3, a_per_state=False,
                    n_state_rows=1, ids=np.array([0], np.int32))
    elif form == "m2g":
        base.update(n_head=4, head_dim=2, n_group=2, a_per_state=False)
    base.update(kw)
    return ssm_inputs.make_problem(**base)


def _vals(p):
    return {k: p.value(k).astype(np.float64).copy() for k in NAMES}


def _loss(p, v, w_y, w_s):
    y, st, _ = oracle.scan_fwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids,
                               dt_softplus=p.dt_softplus, n_threads=1)
    return float(np.sum(y * w_y) + np.sum(st * w_s))


def _grads(p, v, w_y, w_s):
    return oracle.scan_bwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids,
                           w_y, w_s, dt_softplus=p.dt_softplus, n_threads=2)


@pytest.mark.parametrize("form,softplus", [("m1", False), ("m2", False), ("m2g", False),
                                           ("m1", True)])
def test_backward_matches_central_differences(form, softplus):
    """Catches any wrong term, sign or index in every gradient block, including
    the state-row scatter of d_s and the sum over head_dim in d_dt."""
    p = _problem(form, 7 + len(form))
    p.dt_softplus = softplus
    v = _vals(p)
    if softplus:
        v["dt"] = v["dt"] * 6.0 - 2.0   # raw dt on both sides of zero
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
        ana = g["d_" + name]
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(ana, num, rtol=1e-6, atol=1e-7 * scale, err_msg=name)


def _np_forward(v, ids, grp):
    """Independent forward: per-step decays and inputs, then the inclusive
    prefix product of decays; works on complex arrays (for the complex step)."""
    x, dt, A, B, C, D, s = v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["s"]
    S, L, H, P = x.shape
    N = B.shape[3]
    An = A if A.ndim == 2 else A[:, None] * np.ones(N)
    a = np.exp(dt[:, :, :, None, None] * An[None, None, :, None, :]) * np.ones((1, 1, 1, P, 1))
    b = dt[:, :, :, None, None] * x[..., None] * B[:, :, grp, None, :]
    h = s[ids]
    ys = []
    for t in range(L):
        h = a[:, t] * h + b[:, t]
        ys.append(np.einsum("shpn,shn->shp", h, C[:, t, grp]) + D[None, :, None] * x[:, t])
    return np.stack(ys, axis=1), h


@pytest.mark.parametrize("form", ["m1", "m2g"])
def test_adjoint_identity_with_complex_step(form):
    """<dout, J v> equals <J^T dout, v> to rounding, for a random direction v
    in every input at once."""
    p = _problem(form, 31)
    v = _vals(p)
    grp = np.arange(p.n_head) // (p.n_head // p.n_group)
    rng = np.random.default_rng(5)
    direction = {k: rng.standard_normal(v[k].shape) for k in NAMES}
    step = 1e-30
    vc = {k: v[k] + 1j * step * direction[k] for k in NAMES}
    yc, sc = _np_forward(vc, p.ids, grp)
    w_y, w_s = p.value("dy").astype(np.float64), p.value("dstate").astype(np.float64)
    jvp = (np.sum(w_y * yc.imag) + np.sum(w_s * sc.imag)) / step
    g = _grads(p, v, w_y, w_s)
    vjp = sum(np.sum(g["d_" + k] * direction[k]) for k in NAMES)
    assert abs(jvp - vjp) <= 1e-11 * max(1.0, abs(jvp)), (jvp, vjp)
    # and the independent forward agrees with the oracle's
    y, st, _ = oracle.problem_fwd(p)
    yr, sr = _np_forward(v, p.ids, grp)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, sr, rtol=1e-12, atol=1e-13)


def test_zero_upstream_gives_zero_gradients():
    p = _problem("m1", 41)
    v = _vals(p)
    g = _grads(p, v, np.zeros_like(p.value("dy"), dtype=np.float64),
               np.zeros_like(p.value("dstate"), dtype=np.float64))
    for k, arr in g.items():
        assert not np.any(arr), k


def _p1_lti_backward(hidden, inputs, a_bar, b_bar, c_mat, grad_output):
    """The backward equations of the time-invariant diagonal SSM as the page
    states them: dh_t = C^T dy_t + A_bar dh_{t+1}; dA_bar += dh_t h_{t-1};
    dB_bar += dh_t x_t^T; dC += dy_t h_t^T; dx_t = B_bar^T dh_t;
    dh_0 = A_bar dh_1.  hidden holds h_0..h_T (T+1 rows)."""
    T = inputs.shape[0]
    dh_next = np.zeros_like(a_bar)
    ga, gb, gc = np.zeros_like(a_bar), np.zeros_like(b_bar), np.zeros_like(c_mat)
    gx = np.zeros_like(inputs)
    for t in range(T - 1, -1, -1):
        gc += np.outer(grad_output[t], hidden[t + 1])
        dh = c_mat.T @ grad_output[t] + a_bar * dh_next
        ga += dh * hidden[t]
        gb += np.outer(dh, inputs[t])
        gx[t] = b_bar.T @ dh
        dh_next = dh
    return ga, gb, gc, gx, a_bar * dh_next


def test_time_invariant_case_matches_lti_backward():
    """With dt, B and C constant in time and no D, one channel of the
    selective scan is the page's LTI SSM with A_bar = exp(dt A),
    B_bar = dt B (d_model 1) and C constant.  Its gradients map back as
    dA = dA_bar * A_bar * dt, dB_const = dt * dB_bar, dC_const = dC, dh0."""
    p = ssm_inputs.make_problem(n_seqs=1, n_tokens=6, n_head=2, d_state=5, d_conv=0, io="f32",
                                seed=51, h0_std=0.5, A_kind="uniform", A_range=(0.2, 1.5),
                                has_D=False, with_dout=True)
    v = {k: p.value(k).astype(np.float64).copy() for k in ("s", "x", "dt", "A", "B", "C")}
    L, N = 6, 5
    dtc = np.array([0.3, 0.7])
    v["dt"][:] = dtc[None, None, :]
    v["B"][:] = v["B"][:, :1]
    v["C"][:] = v["C"][:, :1]
    dy = p.value("dy").astype(np.float64)
    g = oracle.scan_bwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], None, p.ids,
                        dy, np.zeros((1, 2, 1, N)))
    for h in range(2):
        a_bar = np.exp(dtc[h] * v["A"][h])
        b_bar = (dtc[h] * v["B"][0, 0, 0])[:, None]            # [N][1]
        c_mat = v["C"][0, 0, 0][None, :]                          # [1][N]
        xs = v["x"][0, :, h, :]                                   # [L][1]
        hid = [v["s"][0, h, 0]]
        for t in range(L):
            hid.append(a_bar * hid[-1] + b_bar[:, 0] * xs[t, 0])
        ga, gb, gc, gx, gh0 = _p1_lti_backward(np.array(hid), xs, a_bar, b_bar, c_mat,
                                              dy[0, :, h, :])
        np.testing.assert_allclose(g["d_x"][0, :, h, 0], gx[:, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["d_s"][0, h, 0], gh0, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["d_A"][h], ga * a_bar * dtc[h], rtol=1e-12, atol=1e-14)
    # B and C are shared by both channels: the constant-in-time gradients sum over channels too
    dB_const = np.zeros(N)
    dC_const = np.zeros(N)
    for h in range(2):
        a_bar = np.exp(dtc[h] * v["A"][h])
        b_bar = (dtc[h] * v["B"][0, 0, 0])[:, None]
        c_mat = v["C"][0, 0, 0][None, :]
        xs = v["x"][0, :, h, :]
        hid = [v["s"][0, h, 0]]
        for t in range(L):
            hid.append(a_bar * hid[-1] + b_bar[:, 0] * xs[t, 0])
        ga, gb, gc, gx, gh0 = _p1_lti_backward(np.array(hid), xs, a_bar, b_bar, c_mat,
                                              dy[0, :, h, :])
        dB_const += dtc[h] * gb[:, 0]
        dC_const += gc[0]
    np.testing.assert_allclose(g["d_B"][0, :, 0].sum(axis=0), dB_const, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["d_C"][0, :, 0].sum(axis=0), dC_const, rtol=1e-12, atol=1e-13)
