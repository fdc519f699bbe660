"""GPU parity of ssm_conv_bwd (the ggmlR ssm_conv backward) against the
float64 oracle, called through the C ABI: every element at small ragged
sizes, every element of sampled channels at the 8 x 4096 x 5120 size (each
channel's gradients depend on that channel alone), the empty sequence, the
unaligned-gradient load path, and run-to-run bitwise repeatability."""
import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _check(what, got, want, per_elem=True):
    """d_sx: rtol 1e-4 with an absolute floor of 1e-5 x rms (K-term sums);
    d_w: rtol 1e-4 with a floor of 1e-4 x rms (sums over every token)."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    floor = (1e-5 if per_elem else 1e-4) * max(rms, 1e-30)
    bad = ~(np.abs(got - want) <= floor + 1e-4 * np.abs(want))
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} outside (max err {np.max(np.abs(got - want)):.3g})"


def _problem(seed, n_s, n_t, d_inner, K, io):
    rng = np.random.default_rng(seed)
    sx = ssm_inputs._const(rng.uniform(-1, 1, (n_s, d_inner, K - 1 + n_t)), io)
    w = rng.uniform(-1, 1, (d_inner, K)).astype(np.float32)
    g = rng.uniform(-1, 1, (n_s, n_t, d_inner)).astype(np.float32)
    return sx, w, g


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("K,n_t,d_inner,n_s", [
    (4, 5, 3, 2), (1, 7, 65, 1), (3, 127, 64, 2), (4, 128, 130, 1), (8, 129, 64, 2),
    (4, 300, 200, 3), (2, 1, 1, 1), (5, 1100, 70, 2), (4, 1021, 64, 1)])
def test_conv_bwd_parity(io, silu, K, n_t, d_inner, n_s):
    sx, w, g = _problem(K * 1000 + n_t + d_inner, n_s, n_t, d_inner, K, io)
    d_sx, d_w = ops.conv_bwd(dev(sx), dev(w), dev(g), apply_silu=silu)
    torch.cuda.synchronize()
    o_sx, o_w = oracle.conv_bwd(sx.value, w, g, apply_silu=silu)
    _check("d_sx", host(d_sx), o_sx)
    _check("d_w", host(d_w), o_w, per_elem=False)


def test_conv_bwd_no_tokens():
    sx, w, g = _problem(1, 2, 0, 5, 4, "f32")
    ws = ops.conv_bwd_workspace(2, 0, 5, 4)
    dgrad = torch.full((2 * 5 * 3 + 5 * 4,), float("nan"), device="cuda")
    d_sx, d_w = ops.conv_bwd(dev(sx), dev(w), dev(g), ws=ws, dgrad=dgrad)
    torch.cuda.synchronize()
    assert not host(d_sx).any() and not host(d_w).any()


def test_conv_bwd_unaligned_gradient_rows():
    # dout starts 4 bytes past a 16-byte boundary: the 4-value loads fall back to single floats
    sx, w, g = _problem(2, 2, 70, 64, 4, "f32")
    buf = torch.empty(g.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(g.ravel()).cuda()
    dout = buf[1:].view(g.shape)
    assert dout.data_ptr() % 16 == 4
    d_sx, d_w = ops.conv_bwd(dev(sx), dev(w), dout, apply_silu=True)
    torch.cuda.synchronize()
    o_sx, o_w = oracle.conv_bwd(sx.value, w, g, apply_silu=True)
    _check("d_sx", host(d_sx), o_sx)
    _check("d_w", host(d_w), o_w, per_elem=False)


def test_conv_bwd_full_size_sampled_channels():
    n_s, n_t, d_inner, K = 8, 4096, 5120, 4
    sx, w, g = _problem(0xC5, n_s, n_t, d_inner, K, "bf16")
    d_sx, d_w = ops.conv_bwd(dev(sx), dev(w), dev(g), apply_silu=True)
    torch.cuda.synchronize()
    ch = np.unique(np.concatenate([[0, 63, 64, d_inner - 1],
                                   np.random.default_rng(5).choice(d_inner, 12, replace=False)]))
    o_sx, o_w = oracle.conv_bwd(sx.value[:, ch], w[ch], g[:, :, ch], apply_silu=True)
    hs = torch.as_tensor(ch, device="cuda")
    _check("d_sx", host(d_sx.index_select(1, hs)), o_sx)
    _check("d_w", host(d_w.index_select(0, hs)), o_w, per_elem=False)


def test_conv_bwd_run_to_run_bitwise():
    sx, w, g = _problem(3, 3, 500, 130, 4, "bf16")
    a = [torch.cat([t.reshape(-1) for t in ops.conv_bwd(dev(sx), dev(w), dev(g), apply_silu=True)])
         for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1])
