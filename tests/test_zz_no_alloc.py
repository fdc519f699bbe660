"""selective_scan_fwd_static (no workspace: static device scratch) against
selective_scan_fwd on the same inputs, through the C ABI.  Both run the same
kernels, so their outputs must agree bit for bit.  Two calls in a row, the
second with a smaller input, on the time-chunked path whose carries live in
the scratch; plus the size limit, rejected on the host."""
import numpy as np
import pytest
import torch

import selective_scan_recurrence_amd as ssm
import ssm_inputs
from selective_scan_recurrence_amd import ops

from gpu_util import desc_of, device_inputs

pytestmark = pytest.mark.gpu


def _both(p, chunk):
    t = device_inputs(p)
    d = desc_of(p, chunk=chunk)
    assert ssm.ssm_scan_fwd_plan(d) == "quad_chunked"
    ref = ops.scan_fwd(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"), t["ids"],
                       conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), want_conv_state=True)
    out = torch.full((ssm.ssm_scan_out_bytes(d),), 0x5A, dtype=torch.uint8, device="cuda")
    cso = torch.full((p.n_seqs, p.n_head, p.d_conv - 1), -7.0, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ssm.selective_scan_fwd_static(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                                  t["ids"], t.get("conv_w"), t.get("conv_state"), out, cso, err, None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref.out), "packed y | state differs from selective_scan_fwd"
    assert torch.equal(cso, ref.conv_state), "conv state differs from selective_scan_fwd"
    assert int(err.item()) == 0


def test_static_scratch_matches_workspace_call_twice():
    """A larger chunked call, then a smaller one that reuses the same scratch."""
    big = ssm_inputs.make_problem(n_seqs=4, n_tokens=700, n_head=256, d_state=16, d_conv=4,
                                  io="bf16", seed=0x7A1, h0_std=0.3, conv_state_std=0.5,
                                  n_state_rows=6, ids=np.array([5, 0, 3, 1], np.int32))
    _both(big, chunk=128)
    small = ssm_inputs.make_problem(n_seqs=2, n_tokens=190, n_head=128, d_state=16, d_conv=4,
                                    io="f32", seed=0x7A2, h0_std=0.3, conv_state_std=0.5)
    _both(small, chunk=64)


def test_static_scratch_bad_id_sets_callers_word():
    p = ssm_inputs.make_problem(n_seqs=3, n_tokens=200, n_head=64, d_state=16, d_conv=4, io="f32",
                                seed=0x7A3, h0_std=0.3, n_state_rows=2,
                                ids=np.array([0, 9, 1], np.int32))
    t = device_inputs(p)
    d = desc_of(p, chunk=64)
    out = torch.empty(ssm.ssm_scan_out_bytes(d), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ssm.selective_scan_fwd_static(d, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                                  t["ids"], t.get("conv_w"), None, out, None, err, None)
    torch.cuda.synchronize()
    assert int(err.item()) & ssm.SSM_DEVERR_IDS


def test_static_scratch_rejects_oversized_call():
    # 8 x 2048 x 65536 channels in 256-token chunks needs far more than 32 MiB of carries
    d = ops.make_desc(n_seqs=8, n_tokens=2048, n_head=65536, d_state=16, d_conv=4, chunk=256)
    assert ssm.ssm_scan_workspace_bytes(d, 0) > 32 << 20
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_fwd_static(d, *([None] * 12), None, None)
    assert e.value.status == ssm.SSM_ERR_WORKSPACE
