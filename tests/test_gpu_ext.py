"""GPU parity of selective_scan_fwd_ext (the dt bias, the SiLU(z) gate and
packed variable-length sequences) against ``oracle.scan_fwd_ext``, through
the C ABI, on every kernel path: the Mamba-1 time-split kernel (few rows),
the quad kernels (tiled, untiled, chunked), the Mamba-2 chunked MFMA kernel
and the generic row kernel.  Each case first checks which path its shape
takes."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import ssm_inputs
import selective_scan_recurrence_amd as ssm
from selective_scan_recurrence_amd import ops

from gpu_util import TOL, assert_close, desc_of, dev, device_inputs, host

pytestmark = pytest.mark.gpu

MIX = [0, 1, 2, 70, 133, 200, 64, 31]


def _case(name):
    m1 = dict(d_conv=4, conv_state_std=0.5)
    m2 = dict(a_per_state=False, d_conv=0, A_kind="uniform", A_range=(1.0, 16.0))
    cases = {
        # Mamba-1, d_state 16, few (sequence, channel) rows: the time-split kernel
        "ts_bf16": dict(n_head=128, d_state=16, io="bf16", **m1),
        "ts_f32": dict(n_head=128, d_state=16, io="f32", **m1),
        "ts_bf16_k2": dict(n_head=64, d_state=16, io="bf16", d_conv=2, conv_state_std=0.5),
        "ts_f32_noconv": dict(n_head=48, d_state=16, io="f32", d_conv=0),
        # Mamba-1, d_inner a multiple of 64 and d_state 16, 8 sequences x 64
        # channel blocks: the tiled quad kernel
        "quad_tiled_bf16": dict(n_head=4096, d_state=16, io="bf16", **m1),
        "quad_tiled_f32": dict(n_head=4096, d_state=16, io="f32", **m1),
        "quad_tiled_bf16_chunks": dict(n_head=128, d_state=16, io="bf16", chunk=64, **m1),
        # Mamba-1, d_inner 100 and d_state 10: the untiled quad kernel, chunked
        "quad_untiled_bf16": dict(n_head=100, d_state=10, io="bf16", chunk=48, **m1),
        # Mamba-2 bf16 with head_dim 64, d_state 128: the chunked MFMA kernel
        "ssd_bf16": dict(n_head=4, head_dim=64, d_state=128, n_group=2, io="bf16",
                         bc_std=1.0 / np.sqrt(128.0), **m2),
        "ssd_bf16_p32_n64": dict(n_head=3, head_dim=32, d_state=64, n_group=1, io="bf16",
                                 bc_std=0.125, **m2),
        # generic rows: Mamba-2 in f32; Mamba-1 with d_state 32 (no conv: the row
        # kernel fuses the conv at d_state <= 16); Mamba-1 with two groups and d_conv 3
        "rows_m2_f32": dict(n_head=4, head_dim=4, d_state=32, n_group=2, io="f32", **m2),
        "rows_m1_n32": dict(n_head=40, d_state=32, io="bf16", d_conv=0),
        "rows_m1_g2": dict(n_head=40, d_state=12, n_group=2, io="bf16", d_conv=3, conv_state_std=0.5),
    }
    return cases[name]


# the forward plan each case's shape takes (with the 8-sequence mix)
PLAN = {"ts_bf16": {"time_split"}, "ts_f32": {"time_split"}, "ts_bf16_k2": {"time_split"},
        "ts_f32_noconv": {"time_split"}, "quad_tiled_bf16": {"quad", "quad_relay"},
        "quad_tiled_f32": {"quad", "quad_relay"}, "quad_tiled_bf16_chunks": {"quad_chunked"},
        "quad_untiled_bf16": {"quad_chunked"}, "ssd_bf16": {"ssd"}, "ssd_bf16_p32_n64": {"ssd"},
        "rows_m2_f32": {"rows"}, "rows_m1_n32": {"rows"}, "rows_m1_g2": {"rows"}}


def _plan(p, varlen=True):
    ext = ssm.make_ext(dt_bias=int(p.value("dt_bias") is not None), z=int(p.value("z") is not None),
                       cu_seqlens=int(varlen), total_tokens=p.total_tokens if varlen else 0)
    return ssm.ssm_scan_fwd_plan(desc_of(p), ext)


def _problem(name, lengths=MIX, seed=0x91, with_z=True, bias=True, softplus=True, h0_std=0.3):
    kw = _case(name)
    return ssm_inputs.make_varlen_problem(lengths=lengths, n_state_rows=len(lengths) + 3, seed=seed,
                                          h0_std=h0_std, with_z=with_z, dt_softplus=softplus,
                                          dt_bias_range=(-1.5, 0.5) if bias else None, **kw)


def _run(p, t=None, varlen=True, out=None):
    t = t or device_inputs(p)
    d = desc_of(p)
    cu = dev(p.cu_seqlens) if varlen else None
    ws = ops.workspace(d, False)
    r = ops.scan_fwd_ext(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         dt_bias=t.get("dt_bias"), z=t.get("z"), cu_seqlens=cu,
                         total_tokens=p.total_tokens if varlen else 0, conv_w=t.get("conv_w"),
                         conv_state=t.get("conv_state"), want_conv_state=True, ws=ws, out=out)
    torch.cuda.synchronize()
    return r, ws


def _oracle(p, cu=True, heads=None):
    v = lambda n: None if p.value(n) is None else p.value(n).astype(np.float64)
    h = slice(None) if heads is None else heads
    pk = lambda n: None if v(n) is None else v(n)[0][:, h]
    return oracle.scan_fwd_ext(v("s")[:, h], pk("x"), pk("dt"), v("A")[h], v("B")[0], v("C")[0],
                               None if v("D") is None else v("D")[h], p.ids,
                               cu_seqlens=p.cu_seqlens if cu else None,
                               dt_bias=None if v("dt_bias") is None else v("dt_bias")[h],
                               z=pk("z"), conv_w=None if not p.d_conv else v("conv_w")[h],
                               conv_state=None if not p.d_conv else v("conv_state")[:, h],
                               dt_softplus=p.dt_softplus)


def _z(p):
    z = p.value("z")
    return None if z is None else z[0].astype(np.float64)


def _check_y(io, got, y, z, what):
    if z is None:
        assert_close(got, y, io, f"{what} y")
        return
    rtol, atol = TOL[io]
    scale = np.maximum(1.0, np.abs(z * expit(z)))
    err = np.abs(got - y)
    bad = ~(err <= atol * scale + rtol * np.abs(y))
    if bad.any():
        w = np.unravel_index(np.argmax(err - atol * scale - rtol * np.abs(y)), err.shape)
        raise AssertionError(f"{what} y: {int(bad.sum())}/{bad.size} outside; worst at {w}: "
                             f"got {got[w]!r} want {y[w]!r} gate {z[w] * expit(z[w])!r}")


def _check(p, r, want, what, z=None):
    """y, final states and conv states against the oracle.  With the gate the
    absolute floor of y scales with |SiLU(z)|: the kernel multiplies an fp32
    y, which carries the ungated error, by the gate, so that error is scaled
    by the same factor; the relative term is unchanged."""
    y, st, cso = want
    _check_y(p.io, host(r.y), y, z, what)
    assert_close(host(r.state), st, "f32" if p.io == "f32" else "bf16", f"{what} state")
    if p.d_conv > 1:  # a copy of inputs: exact
        np.testing.assert_array_equal(host(r.conv_state), cso, err_msg=f"{what} conv_state")


@pytest.mark.parametrize("name", ["ts_bf16", "ts_f32", "ts_bf16_k2", "ts_f32_noconv", "quad_tiled_bf16",
                                  "quad_tiled_f32", "quad_tiled_bf16_chunks", "quad_untiled_bf16",
                                  "ssd_bf16", "ssd_bf16_p32_n64", "rows_m2_f32", "rows_m1_n32",
                                  "rows_m1_g2"])
def test_varlen_gate_bias_parity(name):
    """A length mix with empty, 1- and 2-token, ragged and multi-tile
    sequences; z gate, dt bias and softplus on."""
    p = _problem(name)
    assert _plan(p) in PLAN[name]
    r, ws = _run(p)
    _check(p, r, _oracle(p), name, z=_z(p))
    assert ssm.ssm_get_device_error(ws) == 0


@pytest.mark.parametrize("name", ["ssd_bf16", "ssd_bf16_p32_n64", "rows_m2_f32"])
def test_varlen_unit_scale_state(name):
    """Initial states drawn N(0, 1), ten times the workload's scale: the
    carried state enters the chunked MFMA path's C.h product as a bf16 pair,
    so y stays within the same tolerance however large the state is."""
    p = _problem(name, seed=0x97, h0_std=1.0)
    r, _ = _run(p)
    _check(p, r, _oracle(p), f"{name} h0 N(0,1)", z=_z(p))


@pytest.mark.parametrize("name", ["ts_bf16", "quad_tiled_bf16", "ssd_bf16", "rows_m2_f32"])
@pytest.mark.parametrize("with_z,bias", [(False, True), (True, False), (False, False)])
def test_varlen_feature_subsets(name, with_z, bias):
    """Each extra on its own (and neither) on the fused kernels."""
    p = _problem(name, seed=0x92, with_z=with_z, bias=bias, softplus=bias)
    assert _plan(p) in PLAN[name]
    r, _ = _run(p)
    _check(p, r, _oracle(p), f"{name} z={with_z} bias={bias}", z=_z(p))


@pytest.mark.parametrize("name,S", [("ts_bf16", 3), ("quad_tiled_bf16", 8), ("ssd_bf16", 3),
                                    ("rows_m1_g2", 3)])
def test_equal_lengths_with_extras(name, S):
    """Without spans (the [n_seqs][n_tokens] layout), gate and bias only."""
    L = 96
    p = _problem(name, lengths=[L] * S, seed=0x93)
    assert _plan(p, varlen=False) in PLAN[name]
    r, _ = _run(p, varlen=False)
    v = lambda n: None if p.value(n) is None else p.value(n).astype(np.float64)
    sh = lambda a: None if a is None else a[0].reshape((S, L) + a.shape[2:])
    want = oracle.scan_fwd_ext(v("s"), sh(v("x")), sh(v("dt")), v("A"), sh(v("B")), sh(v("C")), v("D"),
                               p.ids, dt_bias=v("dt_bias"), z=sh(v("z")),
                               conv_w=v("conv_w") if p.d_conv else None,
                               conv_state=v("conv_state") if p.d_conv else None,
                               dt_softplus=p.dt_softplus)
    _check(p, r, want, f"{name} equal lengths", z=sh(_z(p)[None]))


def test_ext_without_extras_equals_plain_call():
    """selective_scan_fwd_ext with no extras gives the bytes of selective_scan_fwd."""
    p = ssm_inputs.make_problem(n_seqs=3, n_tokens=130, n_head=128, d_state=16, d_conv=4, io="bf16",
                                seed=0x94, h0_std=0.2, conv_state_std=0.5)
    t = device_inputs(p)
    d = desc_of(p)
    a = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                     conv_w=t["conv_w"], conv_state=t["conv_state"], want_conv_state=True)
    b = ops.scan_fwd_ext(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         conv_w=t["conv_w"], conv_state=t["conv_state"], want_conv_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out) and torch.equal(a.conv_state, b.conv_state)


@pytest.mark.parametrize("name,lengths", [
    ("ts_bf16", [40, 80, 30, 50]), ("quad_tiled_bf16", [40, 80, 30, 50, 20, 10, 5, 7]),
    ("quad_untiled_bf16", [40, 80, 30, 50]), ("ssd_bf16", [40, 80, 30, 50]),
    ("rows_m2_f32", [40, 80, 30, 50])])
def test_invalid_spans(name, lengths):
    """A span longer than desc.n_tokens and one reaching past total_tokens are
    not scanned: NaN final state, y rows untouched, SSM_DEVERR_SEQLENS; the
    valid sequences match the oracle."""
    p = _problem(name, lengths=lengths, seed=0x95)
    p.n_tokens = 64                       # the bound: sequence 1 (80 tokens) is too long
    assert _plan(p) in PLAN[name]
    cu = p.cu_seqlens.copy()              # [0, 40, 120, 150, 200, ...]
    T = int(cu[-1])
    S = len(lengths)
    cu_bad = cu.copy()
    cu_bad[S] = T + 7                     # the last sequence reaches past the packed axis
    t = device_inputs(p)
    d = desc_of(p)
    total, off = ssm.ssm_scan_ext_out_bytes(d, ssm.make_ext(cu_seqlens=1, total_tokens=T))
    out = torch.full((total,), 0x7F, dtype=torch.uint8, device="cuda")
    ws = ops.workspace(d, False)
    r = ops.scan_fwd_ext(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                         dt_bias=t.get("dt_bias"), z=t.get("z"), cu_seqlens=dev(cu_bad), total_tokens=T,
                         conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), want_conv_state=True,
                         ws=ws, out=out)
    torch.cuda.synchronize()
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_SEQLENS
    st = host(r.state)
    assert np.isnan(st[1]).all() and np.isnan(st[S - 1]).all()
    raw = out[:off].cpu().numpy()
    es = 2 if p.io == "bf16" else 4
    row = p.n_head * p.head_dim * es
    for lo, hi in ((cu[1], cu[2]), (cu[S - 1], T)):
        assert (raw[lo * row:hi * row] == 0x7F).all(), "y rows of an invalid span were written"
    want = _oracle(p)
    for i in [0] + list(range(2, S - 1)):
        a, b = cu[i], cu[i + 1]
        _check_y(p.io, host(r.y)[a:b], want[0][a:b], _z(p)[a:b], f"{name} seq {i}")
        assert_close(st[i], want[1][i], "f32" if p.io == "f32" else "bf16", f"{name} seq {i} state")


def test_varlen_full_size_sampled():
    """The 8-sequence, 32768-token, 5120-channel packed batch (a length mix
    with dt bias, softplus and the gate) in the launch configuration bench.py
    times; the oracle on 24 sampled channels, every token."""
    p = ssm_inputs.varlen_config("C9")
    r, ws = _run(p)
    heads = np.sort(np.random.default_rng(9).choice(p.n_head, 24, replace=False))
    y, st, cso = _oracle(p, heads=heads)
    _check_y(p.io, host(r.y)[:, heads], y, _z(p)[:, heads], "C9")
    assert_close(host(r.state)[:, heads], st, "bf16", "C9 state")
    np.testing.assert_array_equal(host(r.conv_state)[:, heads], cso)
    assert ssm.ssm_get_device_error(ws) == 0


@pytest.mark.parametrize("name,S", [("ts_bf16", 3), ("quad_tiled_bf16", 8), ("ssd_bf16", 3),
                                    ("rows_m2_f32", 3)])
def test_all_sequences_empty(name, S):
    """total_tokens = 0 (every span empty, x/dt/B/C/z/y absent): each final state is
    its gathered state row and each conv state its conv-state row; no error."""
    p = _problem(name, lengths=[0] * S, seed=0x96)
    t = device_inputs(p)
    d = desc_of(p)
    d.n_tokens = 8                        # a positive bound; every span is empty
    ws = ops.workspace(d, False)
    x = torch.empty(0, device="cuda")
    r = ops.scan_fwd_ext(d, t["s"], x, x, t["A"], x, x, t.get("D"), t["ids"],
                         dt_bias=t.get("dt_bias"), cu_seqlens=dev(p.cu_seqlens), total_tokens=0,
                         conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), want_conv_state=True,
                         ws=ws)
    torch.cuda.synchronize()
    assert r.y.numel() == 0
    np.testing.assert_array_equal(host(r.state), p.value("s")[p.ids].astype(np.float64))
    if p.d_conv > 1:
        np.testing.assert_array_equal(host(r.conv_state), p.value("conv_state")[p.ids].astype(np.float64))
    assert ssm.ssm_get_device_error(ws) == 0


def test_no_sequences():
    """n_seqs = 0 with spans: nothing is launched and the call succeeds."""
    d = ops.make_desc(n_seqs=0, n_tokens=8, n_head=64, d_state=16, d_conv=4, io="bf16", n_state_rows=1)
    e = torch.empty(0, device="cuda")
    s = torch.zeros(64 * 16, device="cuda")
    A = torch.zeros(64 * 16, device="cuda")
    D = torch.zeros(64, device="cuda")
    w = torch.zeros(64 * 4, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    ws = ops.workspace(d, False)
    ssm.selective_scan_fwd_ext(d, ssm.make_ext(cu_seqlens=cu, total_tokens=0), s, e, e, A, e, e, D, ids,
                               w, None, e, None, ws, ws.numel(), None)
    torch.cuda.synchronize()
