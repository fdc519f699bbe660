"""Seeded random shapes through selective_state_update against the oracle's
decode step, three steps in a row on the same state rows: both forms, the
conv ring (Mamba-1), d_state on and off the fast layouts, f32 and bf16, and
each of dt bias, softplus and the z gate on or off.  Failures name the case."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops

from gpu_util import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu

N_CASES = 16


def _draw(k):
    rng = np.random.default_rng(5000 + k)
    m2 = k % 2 == 1
    S = int(rng.integers(1, 40))
    R = S + int(rng.integers(0, 5))
    io = str(rng.choice(["f32", "bf16"]))
    sp = bool(rng.random() < 0.5)
    ex = dict(with_z=bool(rng.random() < 0.5),
              dt_bias_range=((-1.0, 0.5) if sp else (0.0, 0.5)) if rng.random() < 0.5 else None)
    if m2:
        P = int(rng.choice([4, 32, 64]))
        N = int(rng.choice([12, 16, 64, 128]))
        H = int(rng.choice([2, 3, 4]))
        kw = dict(n_head=H, head_dim=P, d_state=N, n_group=int(rng.choice([g for g in (1, H) if H % g == 0])),
                  a_per_state=False, d_conv=0, A_kind="uniform", A_range=(1.0, 8.0), bc_std=1.0 / np.sqrt(N))
    else:
        N = int(rng.choice([4, 10, 16, 32]))
        H = int(rng.choice([24, 64, 100, 256]))
        K = int(rng.choice([0, 2, 3, 4]))
        kw = dict(n_head=H, d_state=N, d_conv=K, conv_state_std=0.5 if K else None,
                  A_kind="uniform", A_range=(0.5, 8.0))
    return dict(n_seqs=S, n_state_rows=R, io=io, dt_softplus=sp, ids="perm", h0_std=0.3, **kw, **ex)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape_decode(k):
    kw = _draw(k)
    what = f"case {k}: " + ", ".join(f"{a}={b}" for a, b in kw.items())
    p = ssm_inputs.make_decode_problem(seed=6000 + k, **kw)
    d = ops.make_desc(n_seqs=p.n_seqs, n_tokens=1, n_head=p.n_head, head_dim=p.head_dim, d_state=p.d_state,
                      n_group=p.n_group, n_state_rows=p.n_state_rows, a_per_state=p.a_per_state,
                      d_conv=p.d_conv, io=p.io, has_D=p.has_D, dt_softplus=p.dt_softplus)
    t = {n: dev(v) for n, v in p.t.items()}
    t["ids"] = dev(p.ids)
    v = lambda n: None if p.value(n) is None else p.value(n).astype(np.float64)
    S, H, P, G, N = p.n_seqs, p.n_head, p.head_dim, p.n_group, p.d_state
    x, dt = v("x").reshape(S, H, P), v("dt").reshape(S, H)
    B, C = v("B").reshape(S, G, N), v("C").reshape(S, G, N)
    z = None if v("z") is None else v("z").reshape(S, H, P)
    s, cs = v("s"), v("conv_state") if p.d_conv else None
    for step in range(3):   # the same inputs stepped three times: the state and ring carry over
        y = ops.state_update(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                             dt_bias=t.get("dt_bias"), z=t.get("z"), conv_w=t.get("conv_w"),
                             conv_state=t.get("conv_state"))
        torch.cuda.synchronize()
        y_o, s, cs = oracle.state_update(s, x, dt, v("A"), B, C, v("D"), p.ids, dt_bias=v("dt_bias"), z=z,
                                         conv_w=v("conv_w") if p.d_conv else None, conv_state=cs,
                                         dt_softplus=p.dt_softplus)
        rtol, atol = TOL[p.io]
        scale = 1.0 if z is None else np.maximum(1.0, np.abs(z * expit(z)))
        got = host(y)
        bad = ~(np.abs(got - y_o) <= atol * scale + rtol * np.abs(y_o))
        assert not bad.any(), f"{what}: y step {step}: {int(bad.sum())}/{bad.size} outside"
        assert_close(host(t["s"]), s, "f32", f"{what}: state step {step}", tol=(1e-4, 1e-5))
        if p.d_conv > 1:
            assert_close(host(t["conv_state"]), cs, "f32", f"{what}: conv state step {step}", tol=(0, 0))
