"""The relay split of the Mamba-1 forward against the oracle, in full.

When the (sequence, 64-channel block) jobs do not divide evenly over the
compute units, the forward cuts the last jobs into time pieces that hand
their state on through the workspace.  These shapes are sized from the
device's compute-unit count so that the split happens (the plan says
"quad_relay"): half a unit over (2 pieces per split job), a fifth over
(5 pieces), and 3 jobs over (pieces of one tile each), with ragged token
counts, bf16 and f32, with and without the conv, with the dt bias,
softplus and the z gate, and with an invalid id whose NaN state must travel through the
relay.  Every element of y, the final state and the conv state is checked,
and the workspace's error word must stay clear."""
import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
import selective_scan_recurrence_amd as ssm
from selective_scan_recurrence_amd import ops
from tests.gpu_util import assert_close, desc_of, device_inputs, host
from tests.test_gpu_bwd import _compare_all, _run_bwd

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _jobs(kind):
    n = _cus()
    # at least two full jobs per unit: fewer rows take the time-split or
    # chunked kernels instead
    return {"half": 2 * n + n // 2, "fifth": 2 * n + n // 5, "three": 2 * n + 3}[kind]


CASES = {
    # name: (job count kind, sequences, tokens, problem keywords)
    "bf16_conv4_half": ("half", 1, 700, dict(io="bf16", d_conv=4, conv_state_std=0.5)),
    "f32_conv3_fifth": ("fifth", 1, 257, dict(io="f32", d_conv=3, conv_state_std=0.5)),
    "bf16_noconv_three": ("three", 1, 700, dict(io="bf16", d_conv=0)),
    "bf16_conv2_two_seqs_half": ("half", 2, 300, dict(io="bf16", d_conv=2, n_state_rows=4,
                                                      ids=np.array([3, 1], np.int32))),
}


def _problem(name, seed):
    kind, S, L, kw = CASES[name]
    jobs = _jobs(kind)
    assert jobs % S == 0
    return ssm_inputs.make_problem(n_seqs=S, n_tokens=L, n_head=64 * (jobs // S), d_state=16,
                                   seed=seed, h0_std=0.3, **kw)


def _check(p, r, want, what):
    y, st, cso = want
    assert_close(host(r.y), y, p.io, f"{what} y")
    assert_close(host(r.state), st, "f32" if p.io == "f32" else "bf16", f"{what} state")
    if p.d_conv > 1:
        np.testing.assert_array_equal(host(r.conv_state), cso, err_msg=f"{what} conv_state")


@pytest.mark.parametrize("name", sorted(CASES))
def test_relay_parity(gpu, name):
    p = _problem(name, seed=0x3E1 + sorted(CASES).index(name))
    d = desc_of(p)
    assert ssm.ssm_scan_fwd_plan(d) == "quad_relay"
    t = device_inputs(p)
    ws = ops.workspace(d, False)
    r = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                     conv_w=t.get("conv_w"), conv_state=t.get("conv_state"),
                     want_conv_state=True, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "device error word set"
    _check(p, r, oracle.problem_fwd(p), name)
    # a second call on the same workspace: the first must have put every relay
    # flag back to zero, or a piece of the second would start too early
    r2 = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                      conv_w=t.get("conv_w"), conv_state=t.get("conv_state"),
                      want_conv_state=True, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(r2.out, r.out), "second call on the same workspace differs"


@pytest.mark.parametrize("gate", [False, True])
def test_relay_with_bias_softplus_and_gate(gpu, gate):
    """selective_scan_fwd_ext without spans takes the relay too, with the dt
    bias, softplus and (gate) the SiLU(z) output gate."""
    L = 450
    p = ssm_inputs.make_varlen_problem(lengths=[L], n_head=64 * _jobs("half"), d_state=16,
                                       d_conv=4, io="bf16", seed=0x3F0 + gate, h0_std=0.3,
                                       conv_state_std=0.5, dt_softplus=True, with_z=gate,
                                       dt_bias_range=(-1.5, 0.5))
    d = desc_of(p)
    assert ssm.ssm_scan_fwd_plan(d, ssm.make_ext(dt_bias=1, z=int(gate))) == "quad_relay"
    t = device_inputs(p)
    ws = ops.workspace(d, False)
    r = ops.scan_fwd_ext(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         dt_bias=t["dt_bias"], z=t.get("z"), conv_w=t.get("conv_w"),
                         conv_state=t.get("conv_state"), want_conv_state=True, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    v = lambda n: p.value(n).astype(np.float64)
    # one sequence over the whole token axis: the span form of the oracle
    z = v("z")[0] if gate else None
    y, st, cso = oracle.scan_fwd_ext(v("s"), v("x")[0], v("dt")[0], v("A"), v("B")[0], v("C")[0],
                                     v("D"), p.ids, cu_seqlens=np.array([0, L], np.int32),
                                     dt_bias=v("dt_bias"), z=z, conv_w=v("conv_w"),
                                     conv_state=v("conv_state"), dt_softplus=True)
    got = host(r.y).reshape(y.shape)
    if gate:
        # y is gated in fp32 and rounded once: its absolute floor scales with |SiLU(z)|
        scale = np.maximum(1.0, np.abs(z / (1.0 + np.exp(-z))))
        err = np.abs(got - y)
        assert np.all(err <= 1e-3 * scale + 2e-2 * np.abs(y)), float(np.max(err))
    else:
        assert_close(got, y, "bf16", "biased y")
    assert_close(host(r.state), st, "bf16", "relay state")
    np.testing.assert_array_equal(host(r.conv_state), cso)


def test_relay_carries_nan_of_invalid_id(gpu):
    """An invalid id makes that sequence's whole y and state NaN, through every
    piece, and sets SSM_DEVERR_IDS; the other sequence is unaffected."""
    p = ssm_inputs.make_problem(n_seqs=2, n_tokens=300, n_head=64 * (_jobs("half") // 2),
                                d_state=16, d_conv=4, io="bf16", seed=0x3F5, h0_std=0.3,
                                n_state_rows=2, ids=np.array([1, 7], np.int32))
    d = desc_of(p)
    assert ssm.ssm_scan_fwd_plan(d) == "quad_relay"
    t = device_inputs(p)
    ws = ops.workspace(d, False)
    r = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                     conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), ws=ws)
    torch.cuda.synchronize()
    err = int(ws[:4].view(torch.int32).item())
    assert err & ssm.SSM_DEVERR_IDS and not err & ssm.SSM_DEVERR_RELAY
    y, st = host(r.y), host(r.state)
    assert np.isnan(y[1]).all() and np.isnan(st[1]).all()
    v = p.value
    sl = slice(0, 1)
    y_o, st_o, _ = oracle.scan_fwd(v("s"), v("x")[sl], v("dt")[sl], v("A"), v("B")[sl], v("C")[sl],
                                   v("D"), p.ids[sl], conv_w=v("conv_w"),
                                   conv_state=v("conv_state"))
    assert_close(y[0:1], y_o, "bf16", "valid sequence y")
    assert_close(st[0:1], st_o, "bf16", "valid sequence state")



def _no_relay(fn):
    """fn() with the relay split turned off (SSM_RELAY=0, read at every launch)."""
    import os
    old = os.environ.get("SSM_RELAY")
    os.environ["SSM_RELAY"] = "0"
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["SSM_RELAY"]
        else:
            os.environ["SSM_RELAY"] = old


@pytest.mark.parametrize("kind,io,d_conv,L", [("half", "bf16", 4, 600), ("three", "f32", 0, 333)])
def test_forward_relay_bitwise_equals_unsplit(gpu, kind, io, d_conv, L):
    """Pieces start on tile boundaries and pass the fp32 state on, so the
    split grid's y, state and conv state are bitwise those of the unsplit one."""
    p = ssm_inputs.make_problem(n_seqs=1, n_tokens=L, n_head=64 * _jobs(kind), d_state=16,
                                d_conv=d_conv, io=io, seed=0x401, h0_std=0.3,
                                conv_state_std=0.5 if d_conv else None)
    d = desc_of(p)
    assert ssm.ssm_scan_fwd_plan(d) == "quad_relay"
    assert _no_relay(lambda: ssm.ssm_scan_fwd_plan(d)) == "quad"
    t = device_inputs(p)

    def run():
        r = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         conv_w=t.get("conv_w"), conv_state=t.get("conv_state"),
                         want_conv_state=True)
        torch.cuda.synchronize()
        return r

    a, b = run(), _no_relay(run)
    assert torch.equal(a.out, b.out)
    if d_conv > 1:
        assert torch.equal(a.conv_state, b.conv_state)


@pytest.mark.parametrize("S,jobs_kind,L,io,softplus", [
    (8, "half", 256, "bf16", False),   # the 5120-channel layer's job count, two pieces
    (1, "third", 200, "f32", True),    # three pieces, a ragged last block
])
def test_backward_relay_bitwise_equals_unsplit(gpu, S, jobs_kind, L, io, softplus):
    """The backward's reverse-time pass splits the uneven grid into pieces
    that hand on the adjoint and the running dA / dD sums: every gradient is
    bitwise that of the unsplit grid, and matches the oracle."""
    n = _cus()
    jobs = {"half": 2 * n + n // 2, "third": 2 * n + n // 3}[jobs_kind]
    assert jobs % S == 0
    p = ssm_inputs.make_problem(n_seqs=S, n_tokens=L, n_head=64 * (jobs // S), d_state=16, d_conv=0,
                                io=io, seed=0x402 + S, h0_std=0.3, dt_softplus=softplus,
                                with_dout=True, dstate_std=0.5, n_state_rows=S + 1, ids="perm")
    t = device_inputs(p)
    a = _run_bwd(p, t)
    b = _no_relay(lambda: _run_bwd(p, t))
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), f"relay backward {k} differs from the unsplit grid"
    _compare_all(p, a, f"relay backward S={S}")
