"""GPU parity of selective_scan_bwd against the float64 oracle, through the C
ABI.  Gradients are f32 whatever the io dtype: the kernel reads the same
stored inputs as the oracle, so its error is fp32 rounding and accumulation
only.  Per-element gradients (d_x, d_dt) are compared with rtol 1e-4 and an
absolute floor of 1e-5 x rms; channel/token sums (d_A, d_D, d_B, d_C, d_s)
with rtol 1e-4 and a floor of 1e-4 x rms, since a sum of many terms of
either sign carries an absolute error that scales with its terms, not with
its (possibly cancelling) value."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import selective_scan_recurrence_amd as ssm
import ssm_inputs
from selective_scan_recurrence_amd import ops
from tests.gpu_util import desc_of, device_inputs, host

pytestmark = pytest.mark.gpu

PER_ELEM = ("d_x", "d_dt")
SUMS = ("d_s", "d_A", "d_D", "d_B", "d_C")


def _check(name, got, want, floor):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    atol = floor * max(rms, 1e-30)
    err = np.abs(got - want)
    bad = ~(err <= atol + 1e-4 * np.abs(want))
    if bad.any():
        worst = np.unravel_index(np.argmax(err - atol - 1e-4 * np.abs(want)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside (rms {rms:.3g}, atol "
                             f"{atol:.3g}); worst at {worst}: got {got[worst]!r} want {want[worst]!r}")


def _run_bwd(p, t=None, ws=None):
    t = t or device_inputs(p)
    d = desc_of(p)
    dy = t["dy"].reshape(-1).view(torch.uint8)
    dst = t["dstate"].reshape(-1).view(torch.uint8)
    dout = torch.cat([dy, dst])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                        dout, ws=ws)
    torch.cuda.synchronize()
    return g


def _compare_all(p, g, what):
    o = oracle.problem_bwd(p)
    for k in PER_ELEM + SUMS:
        if o.get(k) is None:
            continue
        _check(f"{what} {k}", host(g[k]), o[k], 1e-5 if k in PER_ELEM else 1e-4)


def _small(seed, **kw):
    base = dict(n_seqs=3, n_tokens=37, n_head=70, d_state=16, d_conv=0, io="f32", seed=seed,
                h0_std=0.5, with_dout=True, dstate_std=1.0, A_kind="uniform", A_range=(0.5, 8.0))
    base.update(kw)
    return ssm_inputs.make_problem(**base)


CASES = {
    "f32_ragged": dict(),
    "bf16_ragged": dict(io="bf16"),
    "L1": dict(n_tokens=1),
    "L16": dict(n_tokens=16),
    "L17": dict(n_tokens=17),
    "L100_d128": dict(n_tokens=100, n_head=128),
    "N1": dict(d_state=1),
    "N5": dict(d_state=5),
    "s4d_A": dict(A_kind="s4d"),
    "noD": dict(has_D=False),
    "softplus": dict(dt_softplus=True, dt_shift=0.0),
    "perm_ids": dict(n_state_rows=6, ids="perm"),
    "dup_ids": dict(n_state_rows=4, ids=np.array([2, 2, 0], np.int32)),
    "dstate_zero": dict(dstate_std=0.0),
    "aligned_bf16_tiled": dict(n_head=192, n_tokens=130, io="bf16"),
    "aligned_f32_tiled": dict(n_head=64, n_tokens=77),
    # the prefetched path (64 | channels) around its 8-token block length
    "aligned_L1": dict(n_head=64, n_tokens=1),
    "aligned_L7_bf16_softplus": dict(n_head=64, n_tokens=7, io="bf16", dt_softplus=True, dt_shift=0.0),
    "aligned_L8": dict(n_head=128, n_tokens=8),
    "aligned_L9_bf16": dict(n_head=64, n_tokens=9, io="bf16"),
    "aligned_L24_perm": dict(n_head=64, n_tokens=24, n_state_rows=5, ids="perm"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_edge_case_parity(gpu, case):
    p = _small(zlib.crc32(case.encode()) % 1000, **CASES[case])
    g = _run_bwd(p)
    _compare_all(p, g, case)


@pytest.fixture(scope="module")
def c4_result(gpu):
    """C4 (the backward of the 8 x 4096 x 5120 bf16 scan) run once on the GPU;
    the per-sequence tests below add their oracle shares of the sums over
    sequences (d_A, d_D, d_s) into `partial`."""
    p = ssm_inputs.config("C4")
    g = _run_bwd(p)
    return {"p": p, "g": g, "partial": {}}


def _c4_oracle_seq(p, seq):
    v = p.value
    sl = slice(seq, seq + 1)
    return oracle.scan_bwd(v("s"), v("x")[sl], v("dt")[sl], v("A"), v("B")[sl], v("C")[sl], v("D"),
                           p.ids[sl], v("dy")[sl], v("dstate")[sl])


@pytest.mark.parametrize("seq", range(8))
def test_backward_c4_full_size_every_channel(c4_result, seq):
    """Every channel and token of one sequence of C4: d_x, d_dt and that
    sequence's rows of d_B and d_C against the oracle run on the sequence
    alone."""
    p, g = c4_result["p"], c4_result["g"]
    o = _c4_oracle_seq(p, seq)
    sl = slice(seq, seq + 1)
    for k, floor in (("d_x", 1e-5), ("d_dt", 1e-5), ("d_B", 1e-4), ("d_C", 1e-4)):
        _check(f"C4 sequence {seq} {k}", host(g[k][sl]), o[k], floor)
    c4_result["partial"][seq] = {k: o[k] for k in ("d_A", "d_D", "d_s")}


def test_backward_c4_full_size_sums_over_sequences(c4_result):
    """d_A, d_D and d_s of C4 (sums over all 8 sequences) against the sum of
    the per-sequence oracle gradients (any sequence not done above is run
    here)."""
    p, g, part = c4_result["p"], c4_result["g"], c4_result["partial"]
    for seq in range(p.n_seqs):
        if seq not in part:
            o = _c4_oracle_seq(p, seq)
            part[seq] = {k: o[k] for k in ("d_A", "d_D", "d_s")}
    for k in ("d_A", "d_D", "d_s"):
        want = sum(part[seq][k] for seq in range(p.n_seqs))
        _check(f"C4 {k}", host(g[k]), want, 1e-4)
    for k in ("d_x", "d_dt", "d_B", "d_C"):
        assert bool(torch.isfinite(g[k]).all()), k


def test_backward_no_tokens(gpu):
    p = _small(5, n_tokens=0, n_state_rows=4, ids=np.array([3, 1, 3], np.int32))
    g = _run_bwd(p)
    o = oracle.problem_bwd(p)
    # row 1 has one contributor (exact copy), row 3 two (an fp32 sum), rows 0, 2 none
    np.testing.assert_array_equal(host(g["d_s"])[[0, 1, 2]], o["d_s"][[0, 1, 2]])
    _check("d_s", host(g["d_s"]), o["d_s"], 1e-6)
    assert not host(g["d_A"]).any() and not host(g["d_D"]).any()


def test_backward_run_to_run_bitwise(gpu):
    p = _small(6, n_tokens=200, n_head=128, io="bf16")
    t = device_inputs(p)
    g1 = {k: v.clone() for k, v in _run_bwd(p, t).items()}
    g2 = _run_bwd(p, t)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_bad_id_flag(gpu):
    p = _small(7, n_state_rows=3, ids=np.array([0, 5, 1], np.int32))
    t = device_inputs(p)
    ws = ops.workspace(desc_of(p), True)
    g = _run_bwd(p, t, ws=ws)
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    for k in ("d_x", "d_dt"):
        assert np.isnan(host(g[k])[1]).all(), k
        assert np.isfinite(host(g[k])[[0, 2]]).all(), k
    # the other sequences' own gradients and d_s rows still match the oracle
    keep = [0, 2]
    q = _small(7, n_state_rows=3, ids=np.array([0, 1], np.int32))
    for k in ("x", "dt", "B", "C", "dy", "dstate"):
        q.t[k] = ssm_inputs.Stored(p.t[k].bits[keep], p.t[k].value[keep], p.t[k].dtype)
    o = oracle.problem_bwd(q)
    _check("d_x", host(g["d_x"])[keep], o["d_x"], 1e-5)
    _check("d_s", host(g["d_s"]), o["d_s"], 1e-4)
