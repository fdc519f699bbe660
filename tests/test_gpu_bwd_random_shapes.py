"""Seeded random shapes through selective_scan_bwd (and selective_scan_bwd_conv)
against the oracle's adjoint: the Mamba-1 form (d_state <= 16, one group, f32
or bf16; fixed-order sums, rtol 1e-4 with floors of 1e-5 x rms per element
and 1e-4 x rms for sums), the Mamba-2 form (bf16, head_dim 32/64, d_state
64/128; bf16 MFMA operands, rtol 2e-2 with a floor of 2e-2 x rms), and the
generic kernels (any head_dim, d_state up to 256, groups, either io type, the
fused conv; fp32, the Mamba-1 tolerances), each case with its own length,
heads, ids and softplus choice.  Failures name the case."""
import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops

from gpu_util import desc_of, device_inputs, host

pytestmark = pytest.mark.gpu

N_CASES = 16
N_GENERIC = 16
GRADS = ("d_x", "d_dt", "d_s", "d_A", "d_D", "d_B", "d_C", "d_conv_w", "d_conv_state")
PER_ELEM = ("d_x", "d_dt")


def _draw(k):
    rng = np.random.default_rng(3000 + k)
    m2 = k % 2 == 1
    n_seqs = int(rng.integers(1, 4))
    L = int(rng.integers(1, 260))
    R = n_seqs + int(rng.integers(0, 2))
    ids = rng.permutation(R)[:n_seqs].astype(np.int32)
    if rng.random() < 0.3 and n_seqs > 1:
        ids[1] = ids[0]                      # repeated id: d_s rows accumulate
    sp = bool(rng.random() < 0.5)
    if m2:
        P = int(rng.choice([32, 64]))
        N = int(rng.choice([64, 128]))
        H = int(rng.choice([2, 4]))
        G = int(rng.choice([1, 2]))
        kw = dict(n_head=H, head_dim=P, d_state=N, n_group=G, a_per_state=False, io="bf16",
                  A_kind="uniform", A_range=(1.0, 8.0), bc_std=1.0 / np.sqrt(N), h0_std=0.1)
    else:
        N = int(rng.choice([1, 4, 10, 16]))
        H = int(rng.choice([24, 64, 100, 128]))
        kw = dict(n_head=H, d_state=N, io=str(rng.choice(["f32", "bf16"])), A_kind="uniform",
                  A_range=(0.5, 8.0), h0_std=0.5)
    return dict(n_seqs=n_seqs, n_tokens=L, n_state_rows=R, ids=ids, dt_softplus=sp, d_conv=0,
                has_D=bool(rng.random() < 0.8), **kw), m2


def _draw_generic(k):
    rng = np.random.default_rng(5000 + k)
    n_seqs = int(rng.integers(1, 4))
    L = int(rng.integers(1, 200))
    R = n_seqs + int(rng.integers(0, 2))
    ids = rng.permutation(R)[:n_seqs].astype(np.int32)
    if rng.random() < 0.3 and n_seqs > 1:
        ids[1] = ids[0]
    N = int(rng.choice([1, 3, 7, 16, 24, 64, 100, 256]))
    io = str(rng.choice(["f32", "bf16"]))
    if k % 2 == 0:   # the fused conv (Mamba-1 form, any d_state)
        H = int(rng.choice([8, 40, 96]))
        kw = dict(n_head=H, d_state=N, d_conv=int(rng.choice([2, 3, 4])), io=io,
                  conv_state_std=float(rng.choice([0.0, 0.7])) or None)
    else:            # head_dim > 1 or several groups, either form of A
        H = int(rng.choice([2, 4, 6]))
        P = int(rng.choice([1, 3, 8, 40]))
        G = int(rng.choice([g for g in (1, 2) if H % g == 0]))
        kw = dict(n_head=H, head_dim=P, d_state=N, n_group=G, d_conv=0, io=io,
                  a_per_state=bool(rng.random() < 0.5))
    return dict(n_seqs=n_seqs, n_tokens=L, n_state_rows=R, ids=ids,
                dt_softplus=bool(rng.random() < 0.5), has_D=bool(rng.random() < 0.8),
                A_kind="uniform", A_range=(0.5, 8.0), bc_std=1.0 / np.sqrt(N), h0_std=0.5, **kw)


@pytest.mark.parametrize("k", range(N_GENERIC))
def test_random_shape_bwd_generic(k):
    kw = _draw_generic(k)
    p = ssm_inputs.make_problem(seed=6000 + k, with_dout=True, dstate_std=1.0, **kw)
    what = f"generic case {k}: " + ", ".join(f"{a}={b}" for a, b in kw.items() if a != "ids") + \
           f", ids={list(kw['ids'])}"
    t = device_inputs(p)
    d = desc_of(p)
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout,
                        conv_w=t.get("conv_w"), conv_state=t.get("conv_state"))
    torch.cuda.synchronize()
    o = oracle.problem_bwd(p)
    for name in GRADS:
        if o.get(name) is None:
            continue
        got, want = host(g[name]), np.asarray(o[name], np.float64)
        rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
        per_elem = name == "d_x" or (name == "d_dt" and p.head_dim == 1)
        atol = (1e-5 if per_elem else 1e-4) * max(rms, 1e-30)
        err = np.abs(got - want)
        bad = ~(err <= atol + 1e-4 * np.abs(want))
        assert not bad.any(), f"{what}: {name} {int(bad.sum())}/{bad.size} outside (rms {rms:.3g})"


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape_bwd(k):
    kw, m2 = _draw(k)
    p = ssm_inputs.make_problem(seed=4000 + k, with_dout=True, dstate_std=0.0 if m2 else 1.0, **kw)
    what = f"case {k}: {'m2' if m2 else 'm1'} " + ", ".join(f"{a}={b}" for a, b in kw.items() if a != "ids") + \
           f", ids={list(kw['ids'])}"
    t = device_inputs(p)
    d = desc_of(p)
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout)
    torch.cuda.synchronize()
    o = oracle.problem_bwd(p)
    for name in GRADS:
        if o.get(name) is None:
            continue
        got, want = host(g[name]), np.asarray(o[name], np.float64)
        rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
        if m2:  # d_x, d_B, d_s take only 16-bit operands (M, Lm, G, h_in as bf16 pairs)
            rtol, floor = (1e-3, 1e-3) if name in ("d_x", "d_B", "d_s") else (2e-2, 2e-2)
        else:
            rtol, floor = 1e-4, (1e-5 if name in PER_ELEM else 1e-4)
        atol = floor * max(rms, 1e-30)
        err = np.abs(got - want)
        bad = ~(err <= atol + rtol * np.abs(want))
        assert not bad.any(), f"{what}: {name} {int(bad.sum())}/{bad.size} outside (rms {rms:.3g})"
