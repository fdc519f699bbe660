"""Seeded random shapes through selective_scan_fwd_ext against the oracle:
each case draws the form (Mamba-1 with or without the fused conv, Mamba-2),
the io type, sizes, groups, equal or packed lengths, and which extras are on,
so that every dispatch path of the forward meets shapes the targeted tests
do not.  The draws are fixed by the seed; failures name the case."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops

from gpu_util import TOL, assert_close, desc_of, dev, device_inputs, host

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(k):
    rng = np.random.default_rng(1000 + k)
    form = ["m1conv", "m1", "m2"][k % 3]
    io = "bf16" if rng.random() < 0.6 else "f32"
    n_seqs = int(rng.integers(1, 5))
    if form == "m2":
        head_dim = int(rng.choice([4, 32, 64]))
        d_state = int(rng.choice([16, 64, 128]))
        n_head = int(rng.choice([2, 3, 4]))
        n_group = int(rng.choice([g for g in (1, 2) if n_head % g == 0]))
        kw = dict(n_head=n_head, head_dim=head_dim, d_state=d_state, n_group=n_group, a_per_state=False,
                  d_conv=0, A_kind="uniform", A_range=(1.0, 8.0), bc_std=1.0 / np.sqrt(d_state))
    else:
        d_state = int(rng.choice([4, 10, 16, 32] if form == "m1" else [4, 10, 16]))
        n_head = int(rng.choice([24, 64, 96, 128]))
        kw = dict(n_head=n_head, d_state=d_state)
        if form == "m1conv":
            kw.update(d_conv=int(rng.choice([2, 3, 4])), conv_state_std=0.5)
        else:
            kw.update(d_conv=0)
    varlen = bool(rng.random() < 0.6)
    lengths = rng.integers(0, 150, n_seqs) if varlen else np.full(n_seqs, int(rng.integers(1, 150)))
    extras = dict(with_z=bool(rng.random() < 0.5), softplus=bool(rng.random() < 0.5),
                  bias=bool(rng.random() < 0.5))
    return form, io, kw, varlen, lengths, extras


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape(k):
    form, io, kw, varlen, lengths, ex = _draw(k)
    # dt is a positive step: a bias that could drive dt_raw + bias below zero is
    # drawn only when softplus follows it
    bias_range = ((-1.0, 0.5) if ex["softplus"] else (0.0, 0.5)) if ex["bias"] else None
    p = ssm_inputs.make_varlen_problem(lengths=lengths, n_state_rows=len(lengths) + 1, seed=2000 + k, io=io,
                                       h0_std=0.3, with_z=ex["with_z"], dt_softplus=ex["softplus"],
                                       dt_bias_range=bias_range, **kw)
    what = f"case {k}: {form} {io} {kw} varlen={varlen} lengths={list(lengths)} {ex}"
    t = device_inputs(p)
    d = desc_of(p)
    if not varlen:
        d.n_tokens = int(lengths[0])
    cu = dev(p.cu_seqlens) if varlen else None
    r = ops.scan_fwd_ext(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         dt_bias=t.get("dt_bias"), z=t.get("z"), cu_seqlens=cu,
                         total_tokens=p.total_tokens if varlen else 0, conv_w=t.get("conv_w"),
                         conv_state=t.get("conv_state"), want_conv_state=True)
    torch.cuda.synchronize()
    v = lambda n: None if p.value(n) is None else p.value(n).astype(np.float64)
    S, L = len(lengths), int(lengths[0])
    pk = (lambda a: None if a is None else a[0]) if varlen else \
         (lambda a: None if a is None else a[0].reshape((S, L) + a.shape[2:]))
    y, st, cs = oracle.scan_fwd_ext(v("s"), pk(v("x")), pk(v("dt")), v("A"), pk(v("B")), pk(v("C")), v("D"),
                                    p.ids, cu_seqlens=p.cu_seqlens if varlen else None,
                                    dt_bias=v("dt_bias"), z=pk(v("z")),
                                    conv_w=v("conv_w") if p.d_conv else None,
                                    conv_state=v("conv_state") if p.d_conv else None,
                                    dt_softplus=p.dt_softplus)
    got = host(r.y)
    rtol, atol = TOL[io]
    scale = 1.0 if p.value("z") is None else np.maximum(1.0, np.abs(pk(v("z")) * expit(pk(v("z")))))
    err = np.abs(got - y)
    bad = ~(err <= atol * scale + rtol * np.abs(y))
    assert not bad.any(), f"{what}: y {int(bad.sum())}/{bad.size} outside"
    assert_close(host(r.state), st, "f32" if io == "f32" else "bf16", f"{what}: state")
    if p.d_conv > 1:  # a copy of inputs: exact
        np.testing.assert_array_equal(host(r.conv_state), cs, err_msg=f"{what}: conv state")
