"""GPU parity of the generic backward (every shape outside the specialised
kernels) and of the fused conv + SiLU + scan backward
(selective_scan_bwd_conv), through the C ABI, against the float64 oracle.
The arithmetic is fp32 throughout, so the tolerances are those of the
Mamba-1 backward: rtol 1e-4 with an absolute floor of 1e-5 x rms for the
per-element gradients (d_x, d_dt of one channel) and 1e-4 x rms for sums
(d_dt over a head's channels, d_s, d_A, d_D, d_B, d_C, d_conv_w,
d_conv_state)."""
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

SUMS = ("d_s", "d_A", "d_D", "d_B", "d_C", "d_conv_w", "d_conv_state")


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


def _run(p, t=None, ws=None):
    t = t or device_inputs(p)
    d = desc_of(p)
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout,
                        ws=ws, conv_w=t.get("conv_w"), conv_state=t.get("conv_state"))
    torch.cuda.synchronize()
    return g


def _compare(p, g, what):
    o = oracle.problem_bwd(p)
    for k in ("d_x", "d_dt") + SUMS:
        if o.get(k) is None:
            continue
        per_elem = k == "d_x" or (k == "d_dt" and p.head_dim == 1)
        _check(f"{what} {k}", host(g[k]), o[k], 1e-5 if per_elem else 1e-4)


def _small(seed, **kw):
    base = dict(n_seqs=3, n_tokens=37, n_head=6, d_state=16, d_conv=0, io="f32", seed=seed,
                h0_std=0.5, with_dout=True, dstate_std=1.0, A_kind="uniform", A_range=(0.5, 8.0))
    base.update(kw)
    return ssm_inputs.make_problem(**base)


_M2 = dict(a_per_state=False, A_kind="uniform", A_range=(1.0, 8.0))
_CONV = dict(d_conv=4, head_dim=1, conv_state_std=0.8, n_head=70)

CASES = {
    # the finite-difference shape of the ggmlR page's ssm_scan backward test
    "ggml_fd_shape": dict(n_seqs=1, n_tokens=3, n_head=2, head_dim=2, d_state=3, n_group=1,
                          n_state_rows=1, **_M2),
    "m2_f32_groups_ragged": dict(n_head=4, head_dim=4, d_state=32, n_group=2, **_M2),
    "m2_f32_p64_n128": dict(n_seqs=2, n_tokens=100, n_head=2, head_dim=64, d_state=128, **_M2,
                            bc_std=1 / np.sqrt(128)),
    "m2_bf16_p16_n16_softplus": dict(n_head=3, head_dim=16, d_state=16, io="bf16", **_M2,
                                     dt_softplus=True, dt_shift=0.0),
    "m2_f32_n256_p3_groups": dict(n_seqs=2, n_tokens=20, n_head=6, head_dim=3, d_state=256,
                                  n_group=3, **_M2, bc_std=1 / 16),
    "m2_f32_head_dim_130": dict(n_seqs=1, n_tokens=19, n_head=2, head_dim=130, d_state=8, **_M2),
    "m1_n32": dict(n_head=70, d_state=32),
    "m1_n64_bf16": dict(n_head=40, d_state=64, io="bf16", bc_std=0.25),
    "m1_n5_padded": dict(n_head=33, d_state=5),
    "m1_n17_groups7": dict(n_head=70, d_state=17, n_group=7),
    "m1_a_per_state_p3": dict(n_head=6, head_dim=3, d_state=8, n_group=3),
    "m1_groups2_noD_L1": dict(n_head=64, d_state=16, n_group=2, n_tokens=1, has_D=False),
    "m2_perm_ids": dict(n_head=4, head_dim=8, d_state=16, n_state_rows=6, ids="perm", **_M2),
    "m2_dup_ids": dict(n_head=4, head_dim=8, d_state=16, n_state_rows=2,
                       ids=np.array([1, 1, 0], np.int32), **_M2),
    # the fused conv + SiLU (any d_state)
    "conv4_state_perm": dict(**_CONV, n_state_rows=5, ids="perm"),
    "conv3_dup_ids_softplus": dict(**{**_CONV, "d_conv": 3}, n_state_rows=2,
                                   ids=np.array([1, 1, 0], np.int32), dt_softplus=True, dt_shift=0.0),
    "conv2_bf16_noD": dict(**{**_CONV, "d_conv": 2}, io="bf16", has_D=False),
    "conv4_L2_shorter_than_window": dict(**_CONV, n_tokens=2),
    "conv4_L1": dict(**_CONV, n_tokens=1),
    "conv4_no_conv_state": dict(**{**_CONV, "conv_state_std": None}),
    "conv4_n32_groups2": dict(**_CONV, d_state=32, n_group=2),
    "conv4_s4d_long": {**_CONV, "n_seqs": 2, "n_tokens": 300, "A_kind": "s4d", "n_head": 128},
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_generic_backward_parity(gpu, case):
    p = _small(zlib.crc32(case.encode()) % 1000, **CASES[case])
    _compare(p, _run(p), case)


def test_generic_backward_run_to_run_bitwise(gpu):
    for kw in (CASES["m2_f32_groups_ragged"], CASES["conv4_state_perm"]):
        p = _small(21, **kw)
        t = device_inputs(p)
        g1 = {k: v.clone() for k, v in _run(p, t).items()}
        g2 = _run(p, t)
        for k in g1:
            assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("conv", [False, True])
def test_generic_backward_bad_id(gpu, conv):
    kw = dict(_CONV) if conv else dict(n_head=4, head_dim=8, **_M2)
    kw.update(n_state_rows=3, ids=np.array([0, 5, 1], np.int32))
    p = _small(31, **kw)
    t = device_inputs(p)
    ws = ops.workspace(desc_of(p), True)
    g = _run(p, t, ws=ws)
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    for k in ("d_x", "d_dt"):
        assert np.isnan(host(g[k])[1]).all(), k
        assert np.isfinite(host(g[k])[[0, 2]]).all(), k
    keep = [0, 2]
    q = _small(31, **{**kw, "ids": np.array([0, 1], np.int32)})
    for k in ("x", "dt", "B", "C", "dy", "dstate"):
        q.t[k] = ssm_inputs.Stored(p.t[k].bits[keep], p.t[k].value[keep], p.t[k].dtype)
    q.n_seqs = 2
    o = oracle.problem_bwd(q)
    _check("d_x", host(g["d_x"])[keep], o["d_x"], 1e-5)
    _check("d_s", host(g["d_s"]), o["d_s"], 1e-4)
    if conv:
        _check("d_conv_state", host(g["d_conv_state"]), o["d_conv_state"], 1e-4)


def test_generic_backward_no_tokens(gpu):
    """No tokens: dh_0 is dstate scattered by ids; everything else is zero."""
    p = _small(41, n_tokens=0, n_head=4, head_dim=8, **_M2, n_state_rows=4,
               ids=np.array([3, 1, 3], np.int32))
    g = _run(p)
    o = oracle.problem_bwd(p)
    _check("d_s", host(g["d_s"]), o["d_s"], 1e-6)
    assert not host(g["d_A"]).any() and not host(g["d_D"]).any()


@pytest.fixture(scope="module")
def c10_result(gpu):
    """The backward of the whole 8 x 4096 x 5120 bf16 layer (conv + SiLU +
    scan), run once on the GPU."""
    p = ssm_inputs.config("C10")
    return {"p": p, "g": _run(p), "partial": {}}


def _c10_oracle_seq(p, seq):
    v = p.value
    sl = slice(seq, seq + 1)
    return oracle.scan_bwd(v("s"), v("x")[sl], v("dt")[sl], v("A"), v("B")[sl], v("C")[sl], v("D"),
                           p.ids[sl], v("dy")[sl], v("dstate")[sl], conv_w=v("conv_w"))


@pytest.mark.parametrize("seq", range(8))
def test_fused_backward_full_size_every_channel(c10_result, seq):
    """Every channel and token of one sequence of the 8 x 4096 x 5120 layer:
    d_x (pre-conv), d_dt and that sequence's d_B, d_C rows."""
    p, g = c10_result["p"], c10_result["g"]
    o = _c10_oracle_seq(p, seq)
    sl = slice(seq, seq + 1)
    for k, floor in (("d_x", 1e-5), ("d_dt", 1e-5), ("d_B", 1e-4), ("d_C", 1e-4)):
        _check(f"C10 sequence {seq} {k}", host(g[k][sl]), o[k], floor)
    c10_result["partial"][seq] = {k: o[k] for k in ("d_A", "d_D", "d_s", "d_conv_w", "d_conv_state")}


def test_fused_backward_full_size_sums_over_sequences(c10_result):
    p, g, part = c10_result["p"], c10_result["g"], c10_result["partial"]
    for seq in range(p.n_seqs):
        if seq not in part:
            o = _c10_oracle_seq(p, seq)
            part[seq] = {k: o[k] for k in ("d_A", "d_D", "d_s", "d_conv_w", "d_conv_state")}
    for k in ("d_A", "d_D", "d_s", "d_conv_w", "d_conv_state"):
        want = sum(part[seq][k] for seq in range(p.n_seqs))
        _check(f"C10 {k}", host(g[k]), want, 1e-4)
