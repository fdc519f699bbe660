"""GPU parity of selective_scan_bwd for the Mamba-2 form (scalar A per head,
B/C shared by the heads of a group; bf16 io), the chunked backward on MFMA,
against the float64 oracle through the C ABI.

Tolerance.  The products run with bf16 operands (x, dy, B, C as stored; the
checkpointed state, the carried gradient and the M and Lm tiles as a bf16
value plus a bf16 remainder, about 16 significant bits) and fp32
accumulation.  d_x = M^T dY + diag(w) B G^T + D dY, d_B = Lm^T C + diag(w) X G
and d_s take only such operands and are held to rtol 1e-3 with an absolute
floor of 1e-3 x rms of the oracle's values: over these cases and 210 seeded
random Mamba-2 shapes their worst elements need 5e-5 of (rms + |value|).
d_C also reads the checkpoint, which the forward's recompute forms from
single-bf16 products, and d_dt, d_A through the decay carry a term rounded
once (about 2^-8 relative); they and d_D keep rtol 2e-2 with a 2e-2 x rms
floor, the bf16 tolerance the forward uses with the floor of the sums (their
worst elements need up to 6.9e-3)."""
import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops
from tests.gpu_util import desc_of, device_inputs, dev, host

pytestmark = pytest.mark.gpu

GRADS = ("d_x", "d_dt", "d_s", "d_A", "d_D", "d_B", "d_C")


TIGHT = ("d_x", "d_B", "d_s")  # gradients formed from 16-bit operands only


def _floor(k):
    return 1e-3 if k in TIGHT else 2e-2


def _check(name, got, want, rtol=None, floor=2e-2):
    tight = name.split()[-1] in TIGHT
    if rtol is None:
        rtol = 1e-3 if tight else 2e-2
    if tight:
        floor = min(floor, 1e-3)
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    atol = floor * max(rms, 1e-30)
    err = np.abs(got - want)
    bad = ~(err <= atol + rtol * np.abs(want))
    if bad.any():
        worst = np.unravel_index(np.argmax(err - atol - rtol * np.abs(want)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside (rms {rms:.3g}, atol {atol:.3g}); "
                             f"worst at {worst}: got {got[worst]!r} want {want[worst]!r}")


def _run(p, t=None):
    t = t or device_inputs(p)
    d = desc_of(p)
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout)
    torch.cuda.synchronize()
    return g


def _problem(seed, **kw):
    base = dict(n_seqs=2, n_tokens=200, n_head=4, head_dim=64, d_state=128, n_group=1,
                a_per_state=False, d_conv=0, io="bf16", h0_std=0.1, ids="perm", n_state_rows=3,
                A_kind="uniform", A_range=(1.0, 16.0), bc_std=1.0 / np.sqrt(128.0))
    base.update(kw)
    p = ssm_inputs.make_problem(seed=seed, **base)
    ssm_inputs.add_dout(p, seed + 1)
    return p


CASES = {
    "p64_n128_ragged": dict(),
    "p32_n64_two_groups": dict(n_seqs=1, n_tokens=64, n_head=4, head_dim=32, d_state=64, n_group=2,
                               n_state_rows=1, ids="identity", bc_std=0.125),
    "p64_n64_softplus": dict(n_tokens=130, head_dim=64, d_state=64, n_group=2, dt_softplus=True,
                             bc_std=0.125),
    "p32_n128_one_token": dict(n_seqs=1, n_tokens=1, n_head=2, head_dim=32, n_state_rows=2),
    "p64_n128_no_D_long": dict(n_seqs=1, n_tokens=333, n_head=2, has_D=False, n_state_rows=1,
                               ids="identity"),
    # two sequences start from one state row: their d_s contributions add up
    "p64_n128_dup_ids": dict(n_seqs=3, n_tokens=97, n_head=2, n_state_rows=2,
                             ids=np.array([1, 1, 0], np.int32)),
    # four heads share each of two groups, softplus on, several chunks and a ragged tail
    "p32_n128_groups_softplus": dict(n_seqs=2, n_tokens=200, n_head=8, head_dim=32, n_group=2,
                                     dt_softplus=True, n_state_rows=3),
    # more heads than one 128-head tile of the dt copy, and a ragged 64-token tile
    "p32_n64_136_heads": dict(n_seqs=2, n_tokens=70, n_head=136, head_dim=32, d_state=64, n_group=4,
                              bc_std=0.125, n_state_rows=2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_ssd_bwd_parity(case):
    p = _problem(101 + sorted(CASES).index(case), **CASES[case])
    g = _run(p)
    o = oracle.problem_bwd(p)
    for k in GRADS:
        if o.get(k) is None:
            continue
        _check(f"{case} {k}", host(g[k]), o[k], floor=_floor(k))


def test_ssd_bwd_dstate_seed():
    """A nonzero upstream gradient of the final state enters the last chunk's carry."""
    p = ssm_inputs.make_problem(n_seqs=2, n_tokens=150, n_head=3, head_dim=64, d_state=128,
                                a_per_state=False, d_conv=0, io="bf16", seed=131, h0_std=0.1,
                                ids="perm", n_state_rows=2, A_kind="uniform", A_range=(1.0, 16.0),
                                bc_std=1.0 / np.sqrt(128.0))
    ssm_inputs.add_dout(p, 132, dstate_std=1.0)
    g = _run(p)
    o = oracle.problem_bwd(p)
    for k in GRADS:
        _check(f"dstate {k}", host(g[k]), o[k], floor=_floor(k))


def test_ssd_bwd_bad_id():
    """A sequence whose id is out of range: its d_x and d_dt are NaN, it adds
    nothing to d_s, the error word is set; the other sequence is unaffected."""
    p = _problem(141, n_seqs=2, n_tokens=70, n_head=2, n_state_rows=3)
    t = device_inputs(p)
    bad = p.ids.copy()
    bad[1] = 7
    t["ids"] = dev(bad)
    d = desc_of(p)
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    ws = ops.workspace(d, True)
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout, ws=ws)
    torch.cuda.synchronize()
    import selective_scan_recurrence_amd as ssm
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    assert np.isnan(host(g["d_x"])[1]).all() and np.isnan(host(g["d_dt"])[1]).all()
    # sequence 0 alone, from the oracle
    q = _problem(141, n_seqs=2, n_tokens=70, n_head=2, n_state_rows=3)
    o = oracle.scan_bwd(q.value("s"), q.value("x")[:1], q.value("dt")[:1], q.value("A"), q.value("B")[:1],
                        q.value("C")[:1], q.value("D"), q.ids[:1], q.value("dy")[:1], q.value("dstate")[:1])
    _check("bad-id d_x of the good sequence", host(g["d_x"])[0], o["d_x"][0], floor=1e-2)
    ds = host(g["d_s"])
    _check("bad-id d_s", ds, o["d_s"])


def test_ssd_bwd_full_size_head_subset():
    """The 4 x 4096 x 80 x 64 x 128 workload in the launch configuration bench.py
    times, with dy zero outside three heads: every gradient (d_B and d_C, sums
    over heads, included) then equals the oracle's on those three heads alone."""
    p = ssm_inputs.config("C8")
    heads = np.array([0, 37, 79])
    dy_bits = p.t["dy"].bits.copy()
    mask = np.zeros(p.n_head, bool)
    mask[heads] = True
    dy_bits[:, :, ~mask, :] = 0
    p.t["dy"] = ssm_inputs.Stored(dy_bits, ssm_inputs.bf16_bits_to_f32(dy_bits), "bf16")
    g = _run(p)
    v = p.value
    o = oracle.scan_bwd(v("s")[:, heads], v("x")[:, :, heads], v("dt")[:, :, heads], v("A")[heads],
                        v("B"), v("C"), v("D")[heads], p.ids, v("dy")[:, :, heads], v("dstate")[:, heads])
    _check("C8 d_x", host(g["d_x"])[:, :, heads], o["d_x"], floor=1e-2)
    _check("C8 d_dt", host(g["d_dt"])[:, :, heads], o["d_dt"])
    _check("C8 d_s", host(g["d_s"])[:, heads], o["d_s"])
    _check("C8 d_A", host(g["d_A"])[heads], o["d_A"])
    _check("C8 d_D", host(g["d_D"])[heads], o["d_D"])
    _check("C8 d_B", host(g["d_B"]), o["d_B"])
    _check("C8 d_C", host(g["d_C"]), o["d_C"])


def test_ssd_bwd_run_to_run_bitwise():
    """Every gradient, d_B and d_C (sums over the group's heads) included,
    repeats bit for bit: the head sums are taken in head order."""
    p = _problem(151, n_seqs=2, n_tokens=200, n_head=6, head_dim=64, d_state=128, n_group=2)
    t = device_inputs(p)
    g1 = {k: v.clone() for k, v in _run(p, t).items()}
    g2 = _run(p, t)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


@pytest.fixture(scope="module")
def c8_result():
    """The backward of the 4 x 4096, 80 heads x 64, d_state 128 bf16 scan, run once."""
    p = ssm_inputs.config("C8")
    return {"p": p, "g": _run(p), "partial": {}}


def _c8_oracle_seq(p, seq):
    v = p.value
    sl = slice(seq, seq + 1)
    return oracle.scan_bwd(v("s"), v("x")[sl], v("dt")[sl], v("A"), v("B")[sl], v("C")[sl], v("D"),
                           p.ids[sl], v("dy")[sl], v("dstate")[sl])


@pytest.mark.parametrize("seq", range(4))
def test_ssd_bwd_full_size_every_head(c8_result, seq):
    """Every head, channel and token of one sequence of the full-size workload:
    d_x, d_dt and the sequence's d_B, d_C rows (sums over all 80 heads)."""
    p, g = c8_result["p"], c8_result["g"]
    o = _c8_oracle_seq(p, seq)
    sl = slice(seq, seq + 1)
    for k in ("d_x", "d_dt", "d_B", "d_C"):
        _check(f"C8 sequence {seq} {k}", host(g[k][sl]), o[k], floor=_floor(k))
    c8_result["partial"][seq] = {k: o[k] for k in ("d_A", "d_D", "d_s")}


def test_ssd_bwd_full_size_sums_over_sequences(c8_result):
    p, g, part = c8_result["p"], c8_result["g"], c8_result["partial"]
    for seq in range(p.n_seqs):
        if seq not in part:
            o = _c8_oracle_seq(p, seq)
            part[seq] = {k: o[k] for k in ("d_A", "d_D", "d_s")}
    for k in ("d_A", "d_D", "d_s"):
        _check(f"C8 {k}", host(g[k]), sum(part[seq][k] for seq in range(p.n_seqs)))


def _no_relay(fn):
    """fn() with the relay and round splits turned off (SSM_RELAY=0, read at every launch)."""
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


@pytest.mark.parametrize("n_tokens,softplus", [(1000, False), (1536, True)])
def test_ssd_bwd_round_split_bitwise(n_tokens, softplus):
    """A quarter more (sequence, head) jobs than compute units: the backward
    runs as pieces of whole chunks in rounds (two pieces at 16 chunks, three
    at 24), each handing on the carried gradient and the running sums, so
    every gradient is bitwise that of the unsplit grid (SSM_RELAY=0)."""
    n = torch.cuda.get_device_properties(0).multi_processor_count
    jobs = n + n // 4
    S = 4 if jobs % 4 == 0 else 1
    p = _problem(161 + softplus, n_seqs=S, n_tokens=n_tokens, n_head=jobs // S, n_state_rows=S + 1,
                 dt_softplus=softplus)
    ssm_inputs.add_dout(p, 163, dstate_std=0.5)
    t = device_inputs(p)
    a = {k: v.clone() for k, v in _run(p, t).items()}
    b = _no_relay(lambda: _run(p, t))
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs with the round split"
