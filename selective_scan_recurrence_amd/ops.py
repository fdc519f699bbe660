"""Torch-level convenience over the C ABI: builds descriptors, allocates the
packed outputs and workspaces as torch device tensors, and splits packed
results into views.  Every computation runs in libssm.so's HIP kernels;
torch only provides memory and the stream.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B

IO_DTYPES = {"f32": B.SSM_F32, "bf16": B.SSM_BF16}
TORCH_IO = {B.SSM_F32: torch.float32, B.SSM_BF16: torch.bfloat16}


def make_desc(*, n_seqs, n_tokens, n_head, d_state, head_dim=1, n_group=1, n_state_rows=None,
              a_per_state=True, d_conv=0, chunk=0, io="f32", has_D=True,
              dt_softplus=False) -> B.SsmScanDesc:
    flags = (B.SSM_HAS_D if has_D else 0) | (B.SSM_DT_SOFTPLUS if dt_softplus else 0)
    return B.SsmScanDesc(int(n_seqs), int(n_tokens), int(n_head), int(head_dim), int(d_state),
                         int(n_group), int(n_seqs if n_state_rows is None else n_state_rows),
                         int(bool(a_per_state)), int(d_conv), int(chunk),
                         IO_DTYPES[io] if isinstance(io, str) else int(io), int(flags), 0)


def workspace(desc: B.SsmScanDesc, backward: bool, device="cuda") -> torch.Tensor:
    """A zeroed workspace (its first word is the sticky device-error word)."""
    n = B.ssm_scan_workspace_bytes(desc, int(backward))
    if n == 0:
        raise B.SsmError(B.SSM_ERR_SHAPE, "ssm_scan_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


@dataclass
class FwdResult:
    out: torch.Tensor            # packed bytes: y | state
    y: torch.Tensor              # view [n_seqs][n_tokens][n_head][head_dim], io dtype
    state: torch.Tensor          # view [n_seqs][n_head][head_dim][d_state], f32
    conv_state: Optional[torch.Tensor]


def split_out(desc: B.SsmScanDesc, out: torch.Tensor):
    io = TORCH_IO[desc.io_dtype]
    off = B.ssm_scan_state_offset_bytes(desc)
    n_y = desc.n_seqs * desc.n_tokens * desc.n_head * desc.head_dim
    y = out[:off].view(io)[:n_y].view(desc.n_seqs, desc.n_tokens, desc.n_head, desc.head_dim)
    st = out[off:].view(torch.float32).view(desc.n_seqs, desc.n_head, desc.head_dim, desc.d_state)
    return y, st


def scan_fwd(desc, s, x, dt, A, Bm, Cm, D, ids, conv_w=None, conv_state=None,
             want_conv_state=False, ws=None, out=None, stream=None) -> FwdResult:
    if out is None:
        out = torch.empty(B.ssm_scan_out_bytes(desc), dtype=torch.uint8, device=x.device)
    cso = None
    if want_conv_state and desc.d_conv > 1:
        cso = torch.empty(desc.n_seqs, desc.n_head, desc.d_conv - 1, dtype=torch.float32,
                          device=x.device)
    if ws is None:
        ws = workspace(desc, False, x.device)
    B.selective_scan_fwd(desc, s, x, dt, A, Bm, Cm, D, ids, conv_w, conv_state, out, cso, ws,
                         ws.numel(), stream)
    y, st = split_out(desc, out)
    return FwdResult(out, y, st, cso)


def scan_fwd_ext(desc, s, x, dt, A, Bm, Cm, D, ids, *, dt_bias=None, z=None, cu_seqlens=None,
                 total_tokens=0, conv_w=None, conv_state=None, want_conv_state=False, ws=None,
                 out=None, stream=None) -> FwdResult:
    """selective_scan_fwd_ext.  With cu_seqlens (int32 device [n_seqs+1]) the
    token axis is packed: y is returned as [total_tokens][n_head][head_dim]."""
    ext = B.make_ext(dt_bias, z, cu_seqlens, total_tokens if cu_seqlens is not None else 0)
    total, off = B.ssm_scan_ext_out_bytes(desc, ext)
    if total == 0:
        raise B.SsmError(B.SSM_ERR_SHAPE, "ssm_scan_ext_out_bytes")
    if out is None:
        out = torch.empty(total, dtype=torch.uint8, device=x.device)
    cso = None
    if want_conv_state and desc.d_conv > 1:
        cso = torch.empty(desc.n_seqs, desc.n_head, desc.d_conv - 1, dtype=torch.float32,
                          device=x.device)
    if ws is None:
        ws = workspace(desc, False, x.device)
    B.selective_scan_fwd_ext(desc, ext, s, x, dt, A, Bm, Cm, D, ids, conv_w, conv_state, out, cso,
                             ws, ws.numel(), stream)
    io = TORCH_IO[desc.io_dtype]
    H, P = desc.n_head, desc.head_dim
    n_tok = total_tokens if cu_seqlens is not None else desc.n_seqs * desc.n_tokens
    y = out[:off].view(io)[:n_tok * H * P].view(n_tok, H, P)
    if cu_seqlens is None:
        y = y.view(desc.n_seqs, desc.n_tokens, H, P)
    st = out[off:].view(torch.float32).view(desc.n_seqs, H, P, desc.d_state)
    return FwdResult(out, y, st, cso)


def split_dgrad(desc: B.SsmScanDesc, dgrad: torch.Tensor) -> dict:
    """Views of the packed gradient: d_s, d_x, d_dt, d_A, d_B, d_C, d_D (with
    D), then d_conv_w and d_conv_state (with the fused conv)."""
    total, offs = B.ssm_scan_dgrad_layout(desc)
    S, L, H, P, N, G, R, K = (desc.n_seqs, desc.n_tokens, desc.n_head, desc.head_dim,
                              desc.d_state, desc.n_group, desc.n_state_rows, desc.d_conv)
    shapes = {"d_s": (R, H, P, N), "d_x": (S, L, H, P), "d_dt": (S, L, H),
              "d_A": (H, N) if desc.a_per_state else (H,), "d_B": (S, L, G, N),
              "d_C": (S, L, G, N)}
    if desc.flags & B.SSM_HAS_D:
        shapes["d_D"] = (H,)
    if K > 0:
        shapes["d_conv_w"] = (H, K)
        shapes["d_conv_state"] = (R, H, K - 1)
    res = {}
    off = 0
    for name, shape in shapes.items():
        n = 1
        for v in shape:
            n *= v
        res[name] = dgrad[off:off + 4 * n].view(torch.float32).view(*shape)
        off += 4 * n
    assert off == total, (off, total)
    return res


def scan_bwd(desc, s, x, dt, A, Bm, Cm, D, ids, dout, ws=None, dgrad=None, stream=None,
             conv_w=None, conv_state=None):
    """Returns (packed dgrad bytes, dict of views).  With the fused conv
    (desc.d_conv > 0) conv_w is required and conv_state optional (zeros);
    the call is selective_scan_bwd_conv and d_x is the gradient of the
    pre-conv input."""
    total, _ = B.ssm_scan_dgrad_layout(desc)
    if dgrad is None:
        dgrad = torch.empty(total, dtype=torch.uint8, device=x.device)
    if ws is None:
        ws = workspace(desc, True, x.device)
    if desc.d_conv > 0 or conv_w is not None:
        B.selective_scan_bwd_conv(desc, s, x, dt, A, Bm, Cm, D, ids, conv_w, conv_state, dout, dgrad,
                                  ws, ws.numel(), stream)
    else:
        B.selective_scan_bwd(desc, s, x, dt, A, Bm, Cm, D, ids, dout, dgrad, ws, ws.numel(), stream)
    return dgrad, split_dgrad(desc, dgrad)


def conv_fwd(sx: torch.Tensor, w: torch.Tensor, apply_silu=False, out=None, stream=None):
    """ggml ssm_conv: sx [n_s][d_inner][d_conv-1+n_t], w [d_inner][d_conv] ->
    out [n_s][n_t][d_inner] (sx's dtype)."""
    n_s, d_inner, length = sx.shape
    d_conv = w.shape[1]
    n_t = length - (d_conv - 1)
    io = B.SSM_BF16 if sx.dtype == torch.bfloat16 else B.SSM_F32
    if out is None:
        out = torch.empty(n_s, n_t, d_inner, dtype=sx.dtype, device=sx.device)
    B.ssm_conv_fwd(sx, w, out, n_s, n_t, d_inner, d_conv, io, int(bool(apply_silu)), stream)
    return out


def conv_bwd_workspace(n_s, n_t, d_inner, d_conv, device="cuda") -> torch.Tensor:
    n = B.ssm_conv_bwd_workspace_bytes(n_s, n_t, d_inner, d_conv)
    return torch.empty(max(n, 4), dtype=torch.uint8, device=device)


def conv_bwd(sx: torch.Tensor, w: torch.Tensor, dout: torch.Tensor, apply_silu=False, ws=None,
             dgrad=None, stream=None):
    """Backward of ``conv_fwd``: dout [n_s][n_t][d_inner] (f32) ->
    (d_sx [n_s][d_inner][d_conv-1+n_t], d_w [d_inner][d_conv]), both f32
    views of one packed buffer (d_sx then d_w)."""
    n_s, d_inner, length = sx.shape
    d_conv = w.shape[1]
    n_t = length - (d_conv - 1)
    io = B.SSM_BF16 if sx.dtype == torch.bfloat16 else B.SSM_F32
    if ws is None:
        ws = conv_bwd_workspace(n_s, n_t, d_inner, d_conv, sx.device)
    if dgrad is None:
        dgrad = torch.empty(n_s * d_inner * length + d_inner * d_conv, dtype=torch.float32,
                            device=sx.device)
    B.ssm_conv_bwd(sx, w, dout, dgrad, n_s, n_t, d_inner, d_conv, io, int(bool(apply_silu)), ws,
                   ws.numel(), stream)
    n_sx = n_s * d_inner * length
    return dgrad[:n_sx].view(n_s, d_inner, length), dgrad[n_sx:n_sx + d_inner * d_conv].view(d_inner, d_conv)


def state_update(desc, s, x, dt, A, Bm, Cm, D, ids, *, dt_bias=None, z=None, conv_w=None,
                 conv_state=None, y=None, err=None, stream=None) -> torch.Tensor:
    """One decode token of every sequence (selective_state_update): s and
    conv_state are updated in place; returns y [n_seqs][n_head][head_dim]."""
    if y is None:
        y = torch.empty(desc.n_seqs, desc.n_head, desc.head_dim, dtype=TORCH_IO[desc.io_dtype],
                        device=s.device)
    B.selective_state_update(desc, s, x, dt, dt_bias, A, Bm, Cm, D, z, ids, conv_w, conv_state, y,
                             err, stream)
    return y
