"""The C ABI on the CPU: the library loads, exports every function the header
declares, computes the packed layouts the ggmlR page fixes, and rejects bad
arguments on the host with the documented codes before launching anything.
No test here reaches a kernel launch (there is no GPU in the CPU suite)."""
import ctypes
import json
import os
import re

import pytest

import selective_scan_recurrence_amd as ssm
from selective_scan_recurrence_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "ggml_packed_counts.json")))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ssm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_library_loads_and_exports_every_declared_function():
    lib = ssm.load()
    names = _header_functions()
    assert set(names) == set(ssm.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name
    assert ssm.ssm_version() >= 100


def test_status_strings():
    for code in range(8):
        assert ssm.ssm_status_str(code) != "unknown status"
    assert ssm.ssm_status_str(99) == "unknown status"


def _desc(**kw):
    base = dict(n_seqs=2, n_tokens=2, n_head=3, head_dim=2, d_state=4, n_group=1,
                a_per_state=False, io="f32")
    base.update(kw)
    return ops.make_desc(**base)


def test_packed_forward_counts_match_ggml():
    g = GOLDEN["make_scan_defaults"]
    d = _desc(n_seqs=g["n_seqs"], n_tokens=g["n_seq_tokens"], n_head=g["n_head"],
              head_dim=g["head_dim"], d_state=g["d_state"], n_group=g["n_group"])
    assert ssm.ssm_scan_out_bytes(d) == 4 * g["nelements_packed"]
    assert ssm.ssm_scan_state_offset_bytes(d) == 4 * g["nelements_x"]
    assert ssm.ssm_scan_out_bytes(d) - ssm.ssm_scan_state_offset_bytes(d) == \
        4 * g["nelements_state_block"]


def test_packed_gradient_layout_matches_ggml_order():
    g = GOLDEN["make_scan_defaults"]
    d = _desc(n_seqs=g["n_seqs"], n_tokens=g["n_seq_tokens"], n_head=g["n_head"],
              head_dim=g["head_dim"], d_state=g["d_state"], n_group=g["n_group"], has_D=False)
    total, offs = ssm.ssm_scan_dgrad_layout(d)
    assert total == 4 * g["nelements_scan_back"]
    sizes = [(b - a) // 4 for a, b in zip(offs[:6], offs[1:7])]
    assert sizes == g["scan_back_sizes"]
    assert offs[6] == total          # no d_D block without D
    d2 = _desc(n_seqs=g["n_seqs"], n_tokens=g["n_seq_tokens"], n_head=g["n_head"],
               head_dim=g["head_dim"], d_state=g["d_state"], n_group=g["n_group"], has_D=True)
    total2, offs2 = ssm.ssm_scan_dgrad_layout(d2)
    assert offs2[6] == total and total2 == total + 4 * g["n_head"]


def test_bf16_packing_offsets():
    # y block in bf16, state block in f32 right after it
    d = ops.make_desc(n_seqs=8, n_tokens=4096, n_head=5120, d_state=16, d_conv=4, io="bf16")
    assert ssm.ssm_scan_state_offset_bytes(d) == 335_544_320
    assert ssm.ssm_scan_out_bytes(d) == 335_544_320 + 655_360 * 4
    d3 = ops.make_desc(n_seqs=4, n_tokens=4096, n_head=80, head_dim=64, d_state=128,
                       a_per_state=False, io="bf16")
    assert ssm.ssm_scan_state_offset_bytes(d3) == 167_772_160
    assert ssm.ssm_scan_out_bytes(d3) == 167_772_160 + 2_621_440 * 4


@pytest.mark.parametrize("field,value", [
    ("n_seqs", -1), ("n_tokens", -1), ("n_head", 0), ("head_dim", 0), ("d_state", 0),
    ("d_state", 257), ("n_group", 0), ("n_group", 2), ("n_state_rows", 0), ("a_per_state", 2),
    ("d_conv", -1), ("d_conv", 9), ("chunk", -1), ("flags", 8), ("reserved", 1),
])
def test_invalid_descriptor_rejected(field, value):
    d = _desc()
    setattr(d, field, value)
    assert ssm.ssm_scan_out_bytes(d) == 0
    assert ssm.ssm_scan_workspace_bytes(d, 0) == 0
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_fwd(d, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 20,
                               stream=0)
    assert e.value.status == ssm.SSM_ERR_SHAPE


def test_conv_requires_single_channel_heads():
    d = _desc(d_conv=4, head_dim=2)
    assert ssm.ssm_scan_out_bytes(d) == 0


def test_unknown_dtype_rejected():
    d = _desc()
    d.io_dtype = 7
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_fwd(d, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 20,
                               stream=0)
    assert e.value.status == ssm.SSM_ERR_DTYPE


def _fwd_args(**over):
    a = dict(s=256, x=256, dt=256, A=256, B=256, C=256, D=256, ids=256, conv_w=None,
             conv_state=None, out=256, conv_state_out=None, workspace=256, workspace_bytes=1 << 20)
    a.update(over)
    return a


def _call_fwd(d, a):
    return ssm.selective_scan_fwd(d, a["s"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                                  a["ids"], a["conv_w"], a["conv_state"], a["out"],
                                  a["conv_state_out"], a["workspace"], a["workspace_bytes"],
                                  stream=0)


@pytest.mark.parametrize("name", ["s", "x", "dt", "A", "B", "C", "D", "ids", "out", "workspace"])
def test_null_pointer_rejected(name):
    with pytest.raises(ssm.SsmError) as e:
        _call_fwd(_desc(), _fwd_args(**{name: None}))
    assert e.value.status == ssm.SSM_ERR_NULL


def test_conv_weights_required_with_conv():
    d = _desc(d_conv=4, head_dim=1)
    with pytest.raises(ssm.SsmError) as e:
        _call_fwd(d, _fwd_args())
    assert e.value.status == ssm.SSM_ERR_NULL


def test_small_workspace_rejected():
    d = _desc()
    need = ssm.ssm_scan_workspace_bytes(d, 0)
    assert need >= 256 and need % 256 == 0
    with pytest.raises(ssm.SsmError) as e:
        _call_fwd(d, _fwd_args(workspace_bytes=need - 1))
    assert e.value.status == ssm.SSM_ERR_WORKSPACE


@pytest.mark.parametrize("name,value", [("x", 258), ("s", 258), ("workspace", 512 + 4),
                                        ("out", 258)])
def test_misaligned_pointer_rejected(name, value):
    with pytest.raises(ssm.SsmError) as e:
        _call_fwd(_desc(), _fwd_args(**{name: value}))
    assert e.value.status == ssm.SSM_ERR_ALIGN


def test_backward_rejects_fused_conv():
    d = _desc(d_conv=4, head_dim=1)
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_bwd(d, 256, 256, 256, 256, 256, 256, 256, 256, 256, 256, 256,
                               1 << 20, stream=0)
    assert e.value.status == ssm.SSM_ERR_UNSUPPORTED


def test_conv_argument_checks():
    with pytest.raises(ssm.SsmError) as e:
        ssm.ssm_conv_fwd(None, 256, 256, 1, 4, 2, 3, ssm.SSM_F32, 0, stream=0)
    assert e.value.status == ssm.SSM_ERR_NULL
    with pytest.raises(ssm.SsmError) as e:
        ssm.ssm_conv_fwd(256, 256, 256, 1, 4, 2, 9, ssm.SSM_F32, 0, stream=0)
    assert e.value.status == ssm.SSM_ERR_SHAPE
    with pytest.raises(ssm.SsmError) as e:
        ssm.ssm_conv_fwd(258, 256, 256, 1, 4, 2, 3, ssm.SSM_F32, 0, stream=0)
    assert e.value.status == ssm.SSM_ERR_ALIGN
    with pytest.raises(ssm.SsmError) as e:
        ssm.ssm_conv_fwd(256, 256, 256, 1, 4, 2, 3, 5, 0, stream=0)
    assert e.value.status == ssm.SSM_ERR_DTYPE


def test_fused_backward_argument_checks():
    d = _desc(d_conv=4, head_dim=1)
    ws = ssm.ssm_scan_workspace_bytes(d, 1)
    assert ws >= 256
    # conv weights are required with the fused conv
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_bwd_conv(d, 256, 256, 256, 256, 256, 256, 256, 256, None, None, 256, 256,
                                    256, ws, stream=0)
    assert e.value.status == ssm.SSM_ERR_NULL
    # d_conv 5..8 has no backward kernel
    d5 = _desc(d_conv=5, head_dim=1)
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_bwd_conv(d5, 256, 256, 256, 256, 256, 256, 256, 256, 256, None, 256, 256,
                                    256, 1 << 30, stream=0)
    assert e.value.status == ssm.SSM_ERR_UNSUPPORTED


def test_fused_gradient_layout_appends_conv_blocks():
    d = _desc(d_conv=4, head_dim=1, n_state_rows=3)
    total, offs = ssm.ssm_scan_dgrad_layout(d)
    d0 = _desc(d_conv=0, head_dim=1, n_state_rows=3)
    total0, offs0 = ssm.ssm_scan_dgrad_layout(d0)
    assert offs == offs0
    H, R = d.n_head, d.n_state_rows
    assert total == total0 + 4 * (H * 4 + R * H * 3)


@pytest.mark.parametrize("kw", [dict(a_per_state=False, head_dim=2), dict(d_state=17, head_dim=1),
                                dict(n_group=3, head_dim=1, a_per_state=True),
                                dict(d_state=256, head_dim=3, n_group=3)])
def test_backward_every_forward_shape_has_a_workspace(kw):
    """Shapes outside the specialised kernels take the generic backward: the
    workspace is sized for it (checkpoints, partial slabs) and a short
    workspace is refused before launch."""
    d = _desc(**kw)
    ws = ssm.ssm_scan_workspace_bytes(d, 1)
    assert ws > 256
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_bwd(d, 256, 256, 256, 256, 256, 256, 256, 256, 256, 256, 256, ws - 256,
                               stream=0)
    assert e.value.status == ssm.SSM_ERR_WORKSPACE


def test_conv_bwd_argument_checks():
    n_s, n_t, d_inner, K = 2, 5, 3, 4
    need = ssm.ssm_conv_bwd_workspace_bytes(n_s, n_t, d_inner, K)
    assert need == n_s * 1 * d_inner * K * 4          # one 64-position tile per sequence
    # tiles of 64 positions of sx: 513 positions take 9, 512 take 8
    assert ssm.ssm_conv_bwd_workspace_bytes(1, 510, d_inner, K) == 9 * d_inner * K * 4
    assert ssm.ssm_conv_bwd_workspace_bytes(1, 509, d_inner, K) == 8 * d_inner * K * 4
    assert ssm.ssm_conv_bwd_workspace_bytes(n_s, n_t, d_inner, 9) == 0
    args = dict(n_s=n_s, n_t=n_t, d_inner=d_inner, d_conv=K, io_dtype=ssm.SSM_F32, apply_silu=1,
                workspace=256, workspace_bytes=need, stream=0)
    cases = [
        (dict(sx=None), ssm.SSM_ERR_NULL),
        (dict(dgrad=None), ssm.SSM_ERR_NULL),
        (dict(workspace=None), ssm.SSM_ERR_NULL),
        (dict(workspace_bytes=need - 4), ssm.SSM_ERR_WORKSPACE),
        (dict(d_conv=9), ssm.SSM_ERR_SHAPE),
        (dict(n_t=-1), ssm.SSM_ERR_SHAPE),
        (dict(n_t=(1 << 29) // (d_inner + 64)), ssm.SSM_ERR_SHAPE),   # per-sequence 32-bit offsets
        (dict(io_dtype=7), ssm.SSM_ERR_DTYPE),
        (dict(dout=258), ssm.SSM_ERR_ALIGN),
        (dict(sx=257, io_dtype=ssm.SSM_BF16), ssm.SSM_ERR_ALIGN),
    ]
    for over, status in cases:
        a = dict(sx=256, w=256, dout=256, dgrad=256, **args)
        a.update(over)
        with pytest.raises(ssm.SsmError) as e:
            ssm.ssm_conv_bwd(**a)
        assert e.value.status == status, over


def test_state_update_argument_checks():
    """selective_state_update rejects bad arguments on the host (no launch)."""
    d = ops.make_desc(n_seqs=2, n_tokens=1, n_head=3, d_state=16, d_conv=4, n_state_rows=4)
    base = dict(s=256, x=256, dt=256, dt_bias=None, A=256, B=256, C=256, D=256, z=None, ids=256,
                conv_w=256, conv_state=256, y=256, err=None, stream=0)
    cases = [
        (dict(desc=ops.make_desc(n_seqs=2, n_tokens=2, n_head=3, d_state=16)), ssm.SSM_ERR_SHAPE),
        (dict(desc=ops.make_desc(n_seqs=2, n_tokens=1, n_head=3, d_state=16, head_dim=2,
                                 d_conv=4)), ssm.SSM_ERR_SHAPE),
        (dict(s=None), ssm.SSM_ERR_NULL),
        (dict(ids=None), ssm.SSM_ERR_NULL),
        (dict(y=None), ssm.SSM_ERR_NULL),
        (dict(conv_state=None), ssm.SSM_ERR_NULL),
        (dict(conv_w=None), ssm.SSM_ERR_NULL),
        (dict(D=None), ssm.SSM_ERR_NULL),
        (dict(s=258), ssm.SSM_ERR_ALIGN),
        (dict(z=257), ssm.SSM_ERR_ALIGN),
        (dict(err=258), ssm.SSM_ERR_ALIGN),
        (dict(desc=ops.make_desc(n_seqs=2, n_tokens=1, n_head=3, d_state=16, io=5)),
         ssm.SSM_ERR_DTYPE),
    ]
    for over, status in cases:
        a = dict(desc=d, **base)
        a.update(over)
        with pytest.raises(ssm.SsmError) as e:
            ssm.selective_state_update(**a)
        assert e.value.status == status, over


def test_scan_fwd_ext_argument_checks():
    """selective_scan_fwd_ext rejects bad extras on the host (no launch), and
    sizes its packed result from total_tokens when spans are given."""
    d = ops.make_desc(n_seqs=2, n_tokens=8, n_head=64, d_state=16, d_conv=4, io="bf16")
    ws_bytes = ssm.ssm_scan_workspace_bytes(d, 0)
    base = dict(s=256, x=256, dt=256, A=256, B=256, C=256, D=256, ids=256, conv_w=256,
                conv_state=None, out=256, conv_state_out=None, workspace=256,
                workspace_bytes=ws_bytes, stream=0)
    E = ssm.make_ext
    cases = [
        (E(total_tokens=5), ssm.SSM_ERR_SHAPE),                       # a count without spans
        (E(cu_seqlens=256, total_tokens=-1), ssm.SSM_ERR_SHAPE),
        (E(z=257), ssm.SSM_ERR_ALIGN),                                # z aligned like x (2 bytes)
        (E(dt_bias=258), ssm.SSM_ERR_ALIGN),
        (E(cu_seqlens=258, total_tokens=4), ssm.SSM_ERR_ALIGN),
    ]
    for ext, status in cases:
        with pytest.raises(ssm.SsmError) as e:
            ssm.selective_scan_fwd_ext(d, ext, **base)
        assert e.value.status == status, (ext.z, ext.dt_bias, ext.total_tokens)
    with pytest.raises(ssm.SsmError) as e:
        ssm.selective_scan_fwd_ext(d, E(cu_seqlens=256, total_tokens=3), **dict(base, workspace_bytes=0))
    assert e.value.status == ssm.SSM_ERR_WORKSPACE
    # sizes: y of total_tokens rows then n_seqs states
    n, off = ssm.ssm_scan_ext_out_bytes(d, E(cu_seqlens=256, total_tokens=13))
    assert off == 13 * 64 * 2 and n == off + 2 * 64 * 16 * 4
    assert ssm.ssm_scan_ext_out_bytes(d, None) == (ssm.ssm_scan_out_bytes(d),
                                                   ssm.ssm_scan_state_offset_bytes(d))
    assert ssm.ssm_scan_ext_out_bytes(d, E(total_tokens=3)) == (0, 0)


def test_missing_library_fails_loudly(tmp_path):
    """The binding has no fallback: a package copy without libssm.so raises on
    load() and on the first compute call, naming the missing library."""
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(ssm.__file__)
    dst = tmp_path / "selective_scan_recurrence_amd"
    dst.mkdir()
    for f in os.listdir(src):
        if f.endswith(".py"):
            shutil.copy(os.path.join(src, f), dst / f)
    code = ("import selective_scan_recurrence_amd as m\n"
            "for call in (m.load, lambda: m.ssm_version()):\n"
            "    try:\n"
            "        call()\n"
            "    except RuntimeError as e:\n"
            "        assert 'libssm.so' in str(e) and 'not built' in str(e), e\n"
            "    else:\n"
            "        raise SystemExit('no error without the library')\n"
            "print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                       timeout=120, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr


@pytest.mark.parametrize("kw,want", [
    # the benchmark layers
    (dict(n_seqs=8, n_tokens=2048, n_head=512, head_dim=1, d_state=16, a_per_state=True, d_conv=4),
     "time_split"),
    (dict(n_seqs=8, n_tokens=4096, n_head=5120, head_dim=1, d_state=16, a_per_state=True, d_conv=4,
          io="bf16"), "quad"),
    (dict(n_seqs=4, n_tokens=4096, n_head=80, head_dim=64, d_state=128, io="bf16"), "ssd"),
    # an explicit chunk on the Mamba-1 form asks for the chunked quad kernels
    (dict(n_seqs=8, n_tokens=2048, n_head=512, head_dim=1, d_state=16, a_per_state=True, d_conv=4,
          chunk=256), "quad_chunked"),
    # shapes no specialised kernel takes
    (dict(n_seqs=2, n_tokens=8, n_head=3, head_dim=2, d_state=4), "rows"),
    (dict(n_seqs=2, n_tokens=8, n_head=64, head_dim=1, d_state=32, a_per_state=True), "rows"),
    (dict(n_seqs=0, n_tokens=8, n_head=64, head_dim=1, d_state=16, a_per_state=True,
          n_state_rows=1), "none"),
    # one long f32 sequence of 8192 channels: the time-split kernel, whose
    # buffer descriptors span one 128-token tile (8192 x 4 x 128 bytes), not
    # the 2^32 bytes of the whole sequence
    (dict(n_seqs=1, n_tokens=131072, n_head=8192, head_dim=1, d_state=16, a_per_state=True,
          d_conv=4), "time_split"),
    # a tile of 4M f32 channels no longer fits a descriptor's 31-bit size: the
    # time-split kernel declines it (the quad kernel's 64-token tiles still fit)
    (dict(n_seqs=1, n_tokens=1, n_head=1 << 22, head_dim=1, d_state=16, a_per_state=True,
          d_conv=4), "quad"),
])
def test_forward_plan(kw, want):
    """Which kernel family a forward call runs is decided on the host from the
    descriptor alone (and the alignment of the tensors, here 256 bytes)."""
    base = dict(a_per_state=False, io="f32")
    base.update(kw)
    assert ssm.ssm_scan_fwd_plan(ops.make_desc(**base)) == want


def test_forward_plan_with_extras_and_invalid():
    d = ops.make_desc(n_seqs=8, n_tokens=2048, n_head=512, d_state=16, d_conv=4)
    # the extras ride along on the time-split kernel; an explicit chunk asks
    # for the chunked quad kernels, with or without them
    ext = ssm.make_ext(dt_bias=1, z=1, cu_seqlens=1, total_tokens=100)
    assert ssm.ssm_scan_fwd_plan(d, ext) == "time_split"
    assert ssm.ssm_scan_fwd_plan(d, ssm.make_ext(cu_seqlens=1, total_tokens=100)) == "time_split"
    d.chunk = 256
    assert ssm.ssm_scan_fwd_plan(d, ext) == "quad_chunked"
    bad = ops.make_desc(n_seqs=2, n_tokens=8, n_head=3, head_dim=2, d_state=4)
    bad.d_state = 0
    assert ssm.ssm_scan_fwd_plan(bad) is None
