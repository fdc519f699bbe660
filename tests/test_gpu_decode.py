"""GPU parity of selective_state_update (one decode token per sequence,
states updated in place) against the float64 oracle, through the C ABI:
every element of y, of the updated state rows and of the conv state, over
several consecutive steps, for the Mamba-1 form (with the conv ring) and the
Mamba-2 form, the generic and the 16-states-per-lane kernels, the z gate and
the dt bias with softplus; rows no id names stay bit-exact, a bad id leaves
every row untouched and flags the error word; and the two decode workloads
at full size."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops
from tests.gpu_util import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _desc(p):
    return ops.make_desc(n_seqs=p.n_seqs, n_tokens=1, n_head=p.n_head, head_dim=p.head_dim,
                         d_state=p.d_state, n_group=p.n_group, n_state_rows=p.n_state_rows,
                         a_per_state=p.a_per_state, d_conv=p.d_conv, io=p.io, has_D=p.has_D,
                         dt_softplus=p.dt_softplus)


def _flat(p, name):
    """The decode layout of a one-token operand: x/z [S][H][P], dt [S][H], B/C [S][G][N]."""
    v = p.value(name)
    if v is None:
        return None
    if name in ("x",):
        return v.reshape(p.n_seqs, p.n_head, p.head_dim)
    if name == "dt":
        return v.reshape(p.n_seqs, p.n_head)
    if name in ("B", "C"):
        return v.reshape(p.n_seqs, p.n_group, p.d_state)
    return v


def _oracle_step(p, s, cs):
    return oracle.state_update(s, _flat(p, "x"), _flat(p, "dt"), p.value("A"), _flat(p, "B"),
                               _flat(p, "C"), p.value("D"), p.ids, dt_bias=p.value("dt_bias"),
                               z=p.value("z"), conv_w=p.value("conv_w") if p.d_conv else None,
                               conv_state=cs, dt_softplus=p.dt_softplus)


def _gpu_step(p, t, desc, err=None):
    return ops.state_update(desc, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                            t["ids"], dt_bias=t.get("dt_bias"), z=t.get("z"),
                            conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), err=err)


def _inputs(p):
    t = {k: dev(v) for k, v in p.t.items()}
    t["ids"] = dev(p.ids)
    return t


def _check_steps(p, n_steps=3):
    io = p.io
    t = _inputs(p)
    desc = _desc(p)
    s = p.value("s").astype(np.float64)
    cs = p.value("conv_state").astype(np.float64) if p.d_conv else None
    for step in range(n_steps):
        y = _gpu_step(p, t, desc)
        torch.cuda.synchronize()
        y_o, s, cs = _oracle_step(p, s, cs)
        # the state is held in f32 on both sides: f32 tolerance for it (rows
        # the step reads from a state already rounded once per step)
        assert_close(host(y), y_o, io, f"y step {step}")
        assert_close(host(t["s"]), s, "f32", f"state step {step}", tol=(1e-4, 1e-5))
        if p.d_conv:
            # the ring holds copies of the inputs: exact
            assert np.array_equal(host(t["conv_state"]), cs), f"conv state step {step}"
        # feed the GPU's own state back so that f32 rounding does not compound
        s = host(t["s"])
        if p.d_conv:
            cs = host(t["conv_state"])


CASES = {
    # Mamba-1 with the conv ring, d_state 16 (16 states per lane)
    "m1_k4_n16": dict(n_seqs=5, n_head=70, d_state=16, d_conv=4, n_state_rows=9, ids="perm",
                      h0_std=0.5, conv_state_std=0.5),
    # Mamba-1, d_state 5: the one-lane-per-row kernel
    "m1_k3_n5": dict(n_seqs=3, n_head=33, d_state=5, d_conv=3, n_state_rows=4, ids="perm",
                     h0_std=0.5, conv_state_std=0.5, A_kind="uniform"),
    # Mamba-2: scalar A, two groups, d_state 32 (2 lanes per row) and 128 (8 lanes)
    "m2_n32": dict(n_seqs=3, n_head=6, head_dim=10, d_state=32, n_group=2, a_per_state=False,
                   d_conv=0, n_state_rows=5, ids="perm", h0_std=0.5, A_kind="uniform",
                   A_range=(1.0, 16.0)),
    "m2_n128": dict(n_seqs=2, n_head=4, head_dim=64, d_state=128, n_group=1, a_per_state=False,
                    d_conv=0, n_state_rows=3, ids="perm", h0_std=0.5, A_kind="uniform",
                    A_range=(1.0, 16.0), bc_std=1.0 / np.sqrt(128.0)),
    # d_state 256: 16 lanes per row
    "m2_n256": dict(n_seqs=2, n_head=2, head_dim=4, d_state=256, n_group=2, a_per_state=False,
                    d_conv=0, n_state_rows=2, A_kind="uniform", A_range=(1.0, 16.0)),
}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("epilogue", ["plain", "gate_bias_softplus"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_parity(case, epilogue, io):
    kw = dict(CASES[case])
    extra = {}
    if epilogue != "plain":
        extra = dict(with_z=True, dt_bias_range=(-1.0, 1.0), dt_softplus=True)
    p = ssm_inputs.make_decode_problem(io=io, seed=zlib.crc32(f"{case}-{epilogue}-{io}".encode()) & 0xFFFF, **kw, **extra)
    _check_steps(p)


def test_decode_untouched_rows_and_bad_id():
    p = ssm_inputs.make_decode_problem(n_seqs=3, n_head=20, d_state=16, d_conv=4, n_state_rows=6,
                                       ids="perm", io="f32", seed=7, h0_std=0.5, conv_state_std=0.5)
    t = _inputs(p)
    desc = _desc(p)
    s0, cs0 = host(t["s"]), host(t["conv_state"])
    _gpu_step(p, t, desc)
    torch.cuda.synchronize()
    untouched = np.setdiff1d(np.arange(p.n_state_rows), p.ids)
    assert np.array_equal(host(t["s"])[untouched], s0[untouched])
    assert np.array_equal(host(t["conv_state"])[untouched], cs0[untouched])
    # a bad id: its y is NaN, no row changes, the error word is flagged
    bad = p.ids.copy()
    bad[1] = p.n_state_rows + 3
    t2 = _inputs(p)
    t2["ids"] = dev(bad)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    s1, cs1 = host(t2["s"]), host(t2["conv_state"])
    y = _gpu_step(p, t2, desc, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    assert np.isnan(host(y)[1]).all() and not np.isnan(host(y)[[0, 2]]).any()
    keep = np.setdiff1d(np.arange(p.n_state_rows), bad[[0, 2]])
    assert np.array_equal(host(t2["s"])[keep], s1[keep])
    assert np.array_equal(host(t2["conv_state"])[keep], cs1[keep])


@pytest.mark.parametrize("name", ["C6", "C7"])
def test_decode_workload_full_size(name):
    """Every element of y and of the updated states at the decode workloads'
    full size, in the launch configuration bench.py times."""
    p = ssm_inputs.decode_config(name)
    t = _inputs(p)
    y = _gpu_step(p, t, _desc(p))
    torch.cuda.synchronize()
    cs = p.value("conv_state").astype(np.float64) if p.d_conv else None
    y_o, s_o, cs_o = _oracle_step(p, p.value("s").astype(np.float64), cs)
    assert_close(host(y), y_o, p.io, f"{name} y")
    assert_close(host(t["s"]), s_o, "f32", f"{name} state", tol=(1e-4, 1e-5))
    if p.d_conv:
        assert np.array_equal(host(t["conv_state"]), cs_o)
