"""GPU parity of the fused conv + SiLU + scan backward on the fast Mamba-1
kernels (d_state 16, channels a multiple of 64, 16-byte aligned tensors)
against the float64 oracle, through the C ABI (selective_scan_bwd_conv).

The same calls with a misaligned gradient buffer run the generic kernels;
both must match the oracle, and a relay split of the fast kernel must give
bitwise the gradients of the unsplit grid.  Tolerances are those of the
Mamba-1 backward (fp32 arithmetic): rtol 1e-4 with an absolute floor of
1e-5 x rms for d_x and d_dt and 1e-4 x rms for the sums."""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import selective_scan_recurrence_amd as ssm
import ssm_inputs
from selective_scan_recurrence_amd import ops
from tests.gpu_util import desc_of, device_inputs, host
from tests.test_gpu_bwd_rows import _check, _compare, _run

pytestmark = pytest.mark.gpu

_BASE = dict(n_seqs=3, n_tokens=37, n_head=128, d_state=16, d_conv=4, io="f32", h0_std=0.5,
             with_dout=True, dstate_std=1.0, A_kind="uniform", A_range=(0.5, 8.0),
             conv_state_std=0.8)

CASES = {
    "k4_f32_perm": dict(n_state_rows=5, ids="perm"),
    "k4_bf16": dict(io="bf16", n_head=192),
    "k3_softplus_dup_ids": dict(d_conv=3, dt_softplus=True, n_state_rows=2,
                                ids=np.array([1, 0, 1], np.int32)),
    "k2_bf16_noD": dict(d_conv=2, io="bf16", has_D=False),
    "k4_L8": dict(n_tokens=8),
    "k4_L5_one_partial_block": dict(n_tokens=5),
    "k4_L2": dict(n_tokens=2),
    "k4_L1": dict(n_tokens=1, n_head=64),
    "k4_no_conv_state": dict(conv_state_std=None),
    "k3_long_ragged": dict(d_conv=3, n_seqs=2, n_tokens=301, n_head=64),
}


def _problem(case):
    kw = dict(_BASE)
    kw.update(CASES[case])
    return ssm_inputs.make_problem(seed=zlib.crc32(case.encode()) % 1000, **kw)


def _run_generic(p, t):
    """The same call with the gradient buffer 4 bytes off its alignment: the
    fast kernels need 16-byte rows, so the generic kernels take it."""
    d = desc_of(p)
    total, _ = ssm.ssm_scan_dgrad_layout(d)
    buf = torch.empty(total + 256, dtype=torch.uint8, device="cuda")
    dout = torch.cat([t["dy"].reshape(-1).view(torch.uint8), t["dstate"].reshape(-1).view(torch.uint8)])
    _, g = ops.scan_bwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"], dout,
                        dgrad=buf[4:4 + total], conv_w=t.get("conv_w"), conv_state=t.get("conv_state"))
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", sorted(CASES))
def test_fused_fast_backward_parity(gpu, case):
    p = _problem(case)
    t = device_inputs(p)
    _compare(p, _run(p, t), f"fast {case}")
    _compare(p, _run_generic(p, t), f"generic {case}")


def test_fused_fast_backward_run_to_run_bitwise(gpu):
    p = _problem("k4_bf16")
    t = device_inputs(p)
    g1 = {k: v.clone() for k, v in _run(p, t).items()}
    g2 = _run(p, t)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_fused_fast_backward_bad_id(gpu):
    """An invalid id: that sequence's d_x and d_dt are NaN, the flag is set,
    and the gradients that do not involve it match the oracle without it."""
    p = ssm_inputs.make_problem(seed=77, **{**_BASE, "n_state_rows": 3,
                                            "ids": np.array([0, 5, 1], np.int32)})
    t = device_inputs(p)
    ws = ops.workspace(desc_of(p), True)
    g = _run(p, t, ws=ws)
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    for k in ("d_x", "d_dt"):
        assert np.isnan(host(g[k])[1]).all(), k
        assert np.isfinite(host(g[k])[[0, 2]]).all(), k
    keep = [0, 2]
    q = ssm_inputs.make_problem(seed=77, **{**_BASE, "n_state_rows": 3,
                                            "ids": np.array([0, 1], np.int32), "n_seqs": 2})
    for k in ("x", "dt", "B", "C", "dy", "dstate"):
        q.t[k] = ssm_inputs.Stored(p.t[k].bits[keep], p.t[k].value[keep], p.t[k].dtype)
    o = oracle.problem_bwd(q)
    _check("d_x", host(g["d_x"])[keep], o["d_x"], 1e-5)
    _check("d_s", host(g["d_s"]), o["d_s"], 1e-4)
    _check("d_conv_state", host(g["d_conv_state"]), o["d_conv_state"], 1e-4)


def test_fused_fast_backward_relay_bitwise(gpu):
    """The 5120-channel layer's job count (a relay split on 256 compute
    units): with the split, every gradient is bitwise that of the unsplit
    grid, and both match the oracle."""
    n = torch.cuda.get_device_properties(0).multi_processor_count
    S = 8
    jobs = 2 * n + n // 2
    p = ssm_inputs.make_problem(seed=0x5C1, **{**_BASE, "n_seqs": S, "n_tokens": 45,
                                              "n_head": 64 * (jobs // S), "io": "bf16",
                                              "n_state_rows": S + 2, "ids": "perm"})
    t = device_inputs(p)
    a = {k: v.clone() for k, v in _run(p, t).items()}
    old = os.environ.get("SSM_RELAY")
    os.environ["SSM_RELAY"] = "0"
    try:
        b = _run(p, t)
    finally:
        if old is None:
            del os.environ["SSM_RELAY"]
        else:
            os.environ["SSM_RELAY"] = old
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs with the relay split"
    _compare(p, a, "fused relay")
