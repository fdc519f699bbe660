"""GPU parity of selective_scan_fwd and ssm_conv_fwd against the float64
oracle, called through the C ABI, element by element: the small cases in
full, and the full-size 5120-channel and 80-head layers in full as well
(the latter one sequence per test, so that each oracle run stays short)."""
import numpy as np
import pytest
import torch

import oracle
import ssm_inputs
from selective_scan_recurrence_amd import ops
import zlib

import selective_scan_recurrence_amd as ssm
from tests.gpu_util import assert_close, desc_of, dev, device_inputs, host, run_fwd

pytestmark = pytest.mark.gpu


def _check_full(p, d, r, what):
    y, st, cso = oracle.problem_fwd(p)
    assert_close(host(r.y), y, p.io, f"{what} y")
    assert_close(host(r.state), st, "f32" if p.io == "f32" else "bf16", f"{what} state")
    if p.d_conv > 1:
        np.testing.assert_array_equal(host(r.conv_state), cso)


def _oracle_heads(p, heads):
    """Oracle forward of the given heads only (every sequence, every token)."""
    v = p.value
    heads = np.asarray(heads)
    conv_w = v("conv_w")[heads] if p.d_conv else None
    cs = v("conv_state")[:, heads] if (p.d_conv and "conv_state" in p.t) else None
    A = v("A")[heads]
    grp = oracle.group_of_head(p.n_head, p.n_group)[heads]
    return oracle.scan_fwd(v("s")[:, heads], v("x")[:, :, heads], v("dt")[:, :, heads], A,
                           v("B"), v("C"), v("D")[heads] if p.has_D else None, p.ids,
                           conv_w=conv_w, conv_state=cs, dt_softplus=p.dt_softplus,
                           grp_of_head=grp)


@pytest.mark.parametrize("name", ["C0", "C1"])
def test_config_full_parity(gpu, name):
    p = ssm_inputs.config(name)
    d, r = run_fwd(p)
    _check_full(p, d, r, name)


def test_config_c2_full_size_every_channel(gpu):
    """The 8 x 4096 x 5120 bf16 layer in the launch configuration bench.py
    times: every element of y, of the final state and of the conv state."""
    p = ssm_inputs.config("C2")
    d, r = run_fwd(p, want_conv_state=True)
    y_o, st_o, cso_o = oracle.problem_fwd(p)
    assert_close(host(r.y), y_o, p.io, "C2 y")
    assert_close(host(r.state), st_o, p.io, "C2 state")
    np.testing.assert_array_equal(host(r.conv_state), cso_o)


@pytest.fixture(scope="module")
def c3_result(gpu):
    """C3 (4 x 4096, 80 heads x 64, d_state 128, bf16) run once on the GPU."""
    p = ssm_inputs.config("C3")
    d, r = run_fwd(p)
    return p, r


@pytest.mark.parametrize("seq", range(4))
def test_config_c3_full_size_every_head(c3_result, seq):
    """Every head, channel and token of one sequence of C3 (its own state row
    by the permuted ids) against the oracle run on that sequence alone."""
    p, r = c3_result
    v = p.value
    sl = slice(seq, seq + 1)
    y_o, st_o, _ = oracle.scan_fwd(v("s"), v("x")[sl], v("dt")[sl], v("A"), v("B")[sl], v("C")[sl],
                                   v("D") if p.has_D else None, p.ids[sl],
                                   grp_of_head=oracle.group_of_head(p.n_head, p.n_group))
    assert_close(host(r.y[sl]), y_o, p.io, f"C3 sequence {seq} y")
    assert_close(host(r.state[sl]), st_o, p.io, f"C3 sequence {seq} state")


def _small(seed, **kw):
    base = dict(n_seqs=3, n_tokens=37, n_head=70, d_state=16, d_conv=4, io="f32", seed=seed,
                h0_std=0.5)
    base.update(kw)
    return ssm_inputs.make_problem(**base)


_M2 = dict(d_conv=0, a_per_state=False, A_kind="uniform", io="bf16", bc_std=1 / np.sqrt(128))

CASES = {
    "m1_ragged": dict(),
    "m1_bf16": dict(io="bf16"),
    "m1_L1": dict(n_tokens=1),
    "m1_L2_conv4": dict(n_tokens=2),
    "m1_conv2": dict(d_conv=2),
    "m1_conv3_state": dict(d_conv=3, conv_state_std=1.0),
    "m1_conv4_state_perm": dict(conv_state_std=1.0, n_state_rows=5, ids="perm"),
    "m1_noconv": dict(d_conv=0),
    "m1_noD": dict(has_D=False),
    "m1_softplus": dict(dt_softplus=True, dt_shift=0.0),
    "m1_N1": dict(d_state=1),
    "m1_N5": dict(d_state=5),
    "m1_N17": dict(d_state=17, d_conv=0),
    "m1_N64": dict(d_state=64, d_conv=0, A_kind="uniform"),
    "m1_groups": dict(n_group=7, d_conv=0, A_kind="uniform"),
    "m1_dup_ids": dict(n_state_rows=2, ids=np.array([1, 1, 0], np.int32)),
    # d_inner a multiple of 64 and d_state 16: the LDS-tiled quad path
    "tiled_bf16_ragged": dict(n_head=128, n_tokens=101, io="bf16"),
    "tiled_f32_chunked": dict(n_head=64, n_tokens=300, chunk=64),
    "tiled_bf16_chunked_ragged": dict(n_head=192, n_tokens=333, chunk=128, io="bf16"),
    "tiled_conv_state_perm": dict(n_head=64, n_tokens=70, conv_state_std=1.0, n_state_rows=5,
                                  ids="perm", chunk=32),
    "tiled_L1": dict(n_head=64, n_tokens=1),
    "tiled_L5_noconv": dict(n_head=64, n_tokens=5, d_conv=0),
    "tiled_softplus_noD": dict(n_head=64, n_tokens=77, dt_softplus=True, has_D=False),
    "untiled_chunked": dict(n_head=70, n_tokens=300, chunk=64),
    "m2_small": dict(n_head=5, head_dim=8, d_state=16, d_conv=0, a_per_state=False,
                     A_kind="uniform", n_state_rows=4, ids="perm"),
    "m2_N128_bf16": dict(n_head=4, head_dim=16, d_state=128, d_conv=0, a_per_state=False,
                         A_kind="uniform", io="bf16", bc_std=1 / np.sqrt(128)),
    "m2_N256_groups": dict(n_head=4, head_dim=4, d_state=256, n_group=2, d_conv=0,
                           a_per_state=False, A_kind="uniform", bc_std=1 / 16),
    # d_inner a multiple of 16, few rows, no chunk given: the time-split path
    # (16 channels per workgroup, tiles of 128 tokens)
    "ts_f32_conv4_ragged_perm": dict(n_head=48, n_tokens=300, conv_state_std=1.0, n_state_rows=5,
                                     ids="perm"),
    "ts_bf16_conv3_softplus": dict(n_head=32, n_tokens=129, d_conv=3, dt_softplus=True,
                                   dt_shift=0.0, io="bf16", conv_state_std=1.0),
    "ts_conv2_noD_L128": dict(n_head=16, n_tokens=128, d_conv=2, has_D=False),
    "ts_noconv_L1": dict(n_head=16, n_tokens=1, d_conv=0),
    "ts_conv4_L2": dict(n_head=16, n_tokens=2, conv_state_std=1.0),
    "ts_bf16_long": dict(n_seqs=2, n_head=32, n_tokens=1000, io="bf16"),
    "ts_dup_ids_s4d": dict(n_head=64, n_tokens=200, n_state_rows=2, ids=np.array([1, 1, 0], np.int32)),
    # bf16, head_dim 32/64, d_state 64/128, no conv: the chunked MFMA (SSD) path
    "ssd_P64_N128_ragged_perm": dict(n_head=3, head_dim=64, d_state=128, n_tokens=200,
                                     **_M2, n_state_rows=5, ids="perm"),
    "ssd_P32_N64_groups_L64": dict(n_head=4, head_dim=32, d_state=64, n_group=2, n_tokens=64,
                                   **_M2),
    "ssd_P64_N64_L1": dict(n_head=2, head_dim=64, d_state=64, n_tokens=1, **_M2),
    "ssd_P32_N128_softplus_noD": dict(n_head=3, head_dim=32, d_state=128, n_tokens=130, **_M2,
                                      dt_softplus=True, dt_shift=0.0, has_D=False),
    "ssd_P64_N128_long_noD": dict(n_seqs=2, n_head=2, head_dim=64, d_state=128, n_tokens=1000,
                                  **_M2, has_D=False, h0_std=0.0),
    "ssd_P64_N128_dup_ids": dict(n_head=2, head_dim=64, d_state=128, n_tokens=65, **_M2,
                                 n_state_rows=2, ids=np.array([1, 1, 0], np.int32)),
    "m2_headdim_per_state_A": dict(n_head=6, head_dim=3, d_state=8, d_conv=0,
                                   A_kind="uniform", n_group=3),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_edge_case_parity(gpu, case):
    p = _small(zlib.crc32(case.encode()) % 1000, **CASES[case])
    d, r = run_fwd(p)
    _check_full(p, d, r, case)


def test_empty_inputs(gpu):
    p = _small(7, n_tokens=0, d_conv=0)   # no tokens: the state block is the gathered h0
    d, r = run_fwd(p)
    np.testing.assert_array_equal(host(r.state), p.value("s")[p.ids].astype(np.float64))
    p0 = _small(8, n_seqs=0, n_state_rows=1, d_conv=0)
    d0, r0 = run_fwd(p0)
    assert r0.out.numel() == 0


@pytest.mark.parametrize("n_head", [70, 32])
def test_dt_zero_gathers_state_rows_exactly(gpu, n_head):
    """dt = 0: the final state of sequence i is row ids[i] of s, bit for bit."""
    p = _small(9, d_conv=0, n_state_rows=6, ids=np.array([5, 2, 2], np.int32), n_head=n_head)
    p.t["dt"] = ssm_inputs._const(np.zeros_like(p.value("dt")), p.io)
    s = (np.arange(6 * n_head * 16, dtype=np.float32).reshape(6, n_head, 1, 16) + 1) * 0.25
    p.t["s"] = ssm_inputs._const(s)
    d, r = run_fwd(p)
    np.testing.assert_array_equal(host(r.state), s[p.ids].astype(np.float64))


@pytest.mark.parametrize("n_head", [70, 32])
def test_bad_id_gives_nan_rows_and_sets_flag(gpu, n_head):
    p = _small(10, n_state_rows=3, ids=np.array([1, 3, 0], np.int32), conv_state_std=1.0,
               n_head=n_head)
    t = device_inputs(p)
    ws = ops.workspace(desc_of(p), False)
    d, r = run_fwd(p, t=t, ws=ws)
    y, st = host(r.y), host(r.state)
    assert np.isnan(y[1]).all() and np.isnan(st[1]).all()
    assert np.isfinite(y[[0, 2]]).all() and np.isfinite(st[[0, 2]]).all()
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    # the good sequences still match the oracle
    p.ids = np.array([1, 0], np.int32)
    p.n_seqs = 2
    for k in ("x", "dt", "B", "C"):
        p.t[k] = ssm_inputs.Stored(p.t[k].bits[[0, 2]], p.t[k].value[[0, 2]], p.t[k].dtype)
    y_o, st_o, _ = oracle.problem_fwd(p)
    assert_close(y[[0, 2]], y_o, "f32", "good rows y")
    assert_close(st[[0, 2]], st_o, "f32", "good rows state")


def test_ssd_dt_zero_and_bad_id(gpu):
    """Chunked MFMA path: dt = 0 leaves the gathered state bit for bit; an id
    out of range gives NaN rows for its sequence and sets the flag."""
    p = _small(14, n_head=2, head_dim=64, d_state=128, n_tokens=90, n_state_rows=4,
               ids=np.array([3, 0, 3], np.int32), **_M2)
    p.t["dt"] = ssm_inputs._const(np.zeros_like(p.value("dt")), p.io)
    d, r = run_fwd(p)
    np.testing.assert_array_equal(host(r.state), p.value("s")[p.ids].astype(np.float64))
    q = _small(15, n_head=2, head_dim=32, d_state=64, n_tokens=70, n_state_rows=3,
               ids=np.array([1, 7, 0], np.int32), **_M2)
    t = device_inputs(q)
    ws = ops.workspace(desc_of(q), False)
    d, r = run_fwd(q, t=t, ws=ws)
    y, st = host(r.y), host(r.state)
    assert np.isnan(y[1]).all() and np.isnan(st[1]).all()
    assert ssm.ssm_get_device_error(ws) & ssm.SSM_DEVERR_IDS
    q.ids = np.array([1, 0], np.int32)
    q.n_seqs = 2
    for k in ("x", "dt", "B", "C"):
        q.t[k] = ssm_inputs.Stored(q.t[k].bits[[0, 2]], q.t[k].value[[0, 2]], q.t[k].dtype)
    y_o, st_o, _ = oracle.problem_fwd(q)
    assert_close(y[[0, 2]], y_o, "bf16", "good rows y")
    assert_close(st[[0, 2]], st_o, "bf16", "good rows state")


def test_output_canaries_untouched(gpu):
    p = _small(11, io="bf16")
    d = desc_of(p)
    n = ssm.ssm_scan_out_bytes(d)
    guard = 4096
    buf = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    out = buf[guard:guard + n]
    run_fwd(p, out=out)
    b = buf.cpu().numpy()
    assert (b[:guard] == 0xA5).all() and (b[guard + n:] == 0xA5).all()


def test_run_to_run_bitwise_identical(gpu):
    p = _small(12, n_tokens=300, io="bf16")
    t = device_inputs(p)
    _, r1 = run_fwd(p, t=t)
    _, r2 = run_fwd(p, t=t)
    assert torch.equal(r1.out, r2.out)


def test_zero_operands_give_zero_output(gpu):
    p = _small(13, d_conv=0)
    for k in ("s", "x", "dt", "A", "B", "C", "D"):
        p.t[k] = ssm_inputs._const(np.zeros_like(p.value(k)), p.t[k].dtype)
    d, r = run_fwd(p)
    assert not bool(r.out.any())


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d_conv,n_t,d_inner,n_s,silu", [
    (3, 4, 2, 1, False), (4, 5, 3, 2, True), (4, 130, 200, 3, False), (1, 7, 65, 1, True),
    (8, 64, 64, 2, True), (4, 1, 1, 1, False)])
def test_ssm_conv_parity(gpu, io, d_conv, n_t, d_inner, n_s, silu):
    rng = np.random.default_rng(d_conv * 1000 + n_t)
    sx = ssm_inputs._const(rng.uniform(-1, 1, (n_s, d_inner, d_conv - 1 + n_t)), io)
    w = rng.uniform(-1, 1, (d_inner, d_conv)).astype(np.float32)
    got = ops.conv_fwd(dev(sx), dev(w), apply_silu=silu)
    torch.cuda.synchronize()
    want = oracle.conv_fwd(sx.value, w, apply_silu=silu)
    assert_close(host(got), want, io, "ssm_conv")


def test_ssm_conv_full_size(gpu):
    """The standalone conv + SiLU over the 8 x 4096 x 5120 bf16 activations, in
    the launch configuration bench.py times: every output element."""
    c = ssm_inputs.conv_config("C11")
    got = ops.conv_fwd(dev(c.sx), dev(c.w), apply_silu=c.apply_silu)
    torch.cuda.synchronize()
    want = oracle.conv_fwd(c.sx.value, c.w.value, apply_silu=c.apply_silu)
    assert_close(host(got), want, c.io, "ssm_conv C11")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d_inner,n_t", [(72, 130), (8, 64), (136, 65)])
def test_ssm_conv_row_pieces(gpu, io, d_inner, n_t):
    """Channel counts that are multiples of 8 but not of 64 (the 16-byte row
    stores of the last channel block stop at d_inner), with ragged tiles."""
    rng = np.random.default_rng(d_inner + n_t)
    sx = ssm_inputs._const(rng.uniform(-1, 1, (2, d_inner, 3 + n_t)), io)
    w = rng.uniform(-1, 1, (d_inner, 4)).astype(np.float32)
    got = ops.conv_fwd(dev(sx), dev(w), apply_silu=True)
    torch.cuda.synchronize()
    assert_close(host(got), oracle.conv_fwd(sx.value, w, apply_silu=True), io, "ssm_conv rows")
