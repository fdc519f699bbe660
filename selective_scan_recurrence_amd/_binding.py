"""ctypes binding of libssm.so: the C ABI of include/ssm.h under the same
names, with argument marshalling only.  Tensors may be passed as torch
tensors (their data_ptr is used), raw integer addresses, or None for NULL.
Every compute call raises SsmError on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm.so")

SSM_OK, SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_UNSUPPORTED, \
    SSM_ERR_WORKSPACE, SSM_ERR_ALIGN, SSM_ERR_HIP = range(8)
SSM_F32, SSM_BF16 = 0, 1
SSM_HAS_D, SSM_DT_SOFTPLUS = 1, 2
SSM_DEVERR_IDS, SSM_DEVERR_SEQLENS, SSM_DEVERR_RELAY = 1, 2, 4

EXPORTS = ("ssm_status_str", "ssm_version", "ssm_scan_out_bytes", "ssm_scan_state_offset_bytes",
           "ssm_scan_dgrad_layout", "ssm_scan_workspace_bytes", "ssm_conv_fwd",
           "ssm_conv_bwd_workspace_bytes", "ssm_conv_bwd", "selective_scan_fwd",
           "selective_scan_bwd", "selective_state_update", "ssm_get_device_error",
           "ssm_scan_ext_out_bytes", "selective_scan_fwd_ext", "ssm_scan_fwd_plan",
           "selective_scan_fwd_static", "selective_scan_bwd_conv")


class SsmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({ssm_status_str(status)})")


class SsmScanDesc(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
                ("n_head", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("n_group", ctypes.c_int64),
                ("n_state_rows", ctypes.c_int64), ("a_per_state", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class SsmScanExt(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("cu_seqlens", ctypes.c_void_p), ("total_tokens", ctypes.c_int64)]


_lib = None
_lock = threading.Lock()


def load():
    """Loads libssm.so (built in-tree by selective_scan_recurrence_amd.build).
    Raises if it is missing: there is no fallback path."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m selective_scan_recurrence_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        D = ctypes.POINTER(SsmScanDesc)
        lib.ssm_status_str.argtypes, lib.ssm_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        lib.ssm_version.argtypes, lib.ssm_version.restype = [], ctypes.c_int
        for fn in ("ssm_scan_out_bytes", "ssm_scan_state_offset_bytes"):
            getattr(lib, fn).argtypes, getattr(lib, fn).restype = [D], SZ
        lib.ssm_scan_dgrad_layout.argtypes = [D, ctypes.POINTER(SZ * 7)]
        lib.ssm_scan_dgrad_layout.restype = SZ
        lib.ssm_scan_workspace_bytes.argtypes = [D, ctypes.c_int]
        lib.ssm_scan_workspace_bytes.restype = SZ
        lib.ssm_conv_fwd.argtypes = [P, P, P, I64, I64, I64, I32, I32, I32, P]
        lib.ssm_conv_fwd.restype = ctypes.c_int
        lib.ssm_conv_bwd_workspace_bytes.argtypes = [I64, I64, I64, I32]
        lib.ssm_conv_bwd_workspace_bytes.restype = SZ
        lib.ssm_conv_bwd.argtypes = [P, P, P, P, I64, I64, I64, I32, I32, I32, P, SZ, P]
        lib.ssm_conv_bwd.restype = ctypes.c_int
        lib.selective_scan_fwd.argtypes = [D] + [P] * 13 + [SZ, P]
        lib.selective_scan_fwd.restype = ctypes.c_int
        lib.selective_scan_bwd.argtypes = [D] + [P] * 11 + [SZ, P]
        lib.selective_scan_bwd.restype = ctypes.c_int
        lib.selective_scan_bwd_conv.argtypes = [D] + [P] * 13 + [SZ, P]
        lib.selective_scan_bwd_conv.restype = ctypes.c_int
        lib.selective_state_update.argtypes = [D] + [P] * 15
        lib.selective_state_update.restype = ctypes.c_int
        E = ctypes.POINTER(SsmScanExt)
        lib.ssm_scan_ext_out_bytes.argtypes = [D, E, ctypes.POINTER(SZ)]
        lib.ssm_scan_ext_out_bytes.restype = SZ
        lib.selective_scan_fwd_ext.argtypes = [D, E] + [P] * 13 + [SZ, P]
        lib.selective_scan_fwd_ext.restype = ctypes.c_int
        lib.selective_scan_fwd_static.argtypes = [D] + [P] * 13 + [P]
        lib.selective_scan_fwd_static.restype = ctypes.c_int
        lib.ssm_scan_fwd_plan.argtypes = [D, E]
        lib.ssm_scan_fwd_plan.restype = ctypes.c_char_p
        lib.ssm_get_device_error.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
        lib.ssm_get_device_error.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc != SSM_OK:
        raise SsmError(rc, where)
    return rc


def ssm_status_str(status: int) -> str:
    return load().ssm_status_str(int(status)).decode()


def ssm_version() -> int:
    return load().ssm_version()


def ssm_scan_out_bytes(desc: SsmScanDesc) -> int:
    return load().ssm_scan_out_bytes(ctypes.byref(desc))


def ssm_scan_state_offset_bytes(desc: SsmScanDesc) -> int:
    return load().ssm_scan_state_offset_bytes(ctypes.byref(desc))


def ssm_scan_dgrad_layout(desc: SsmScanDesc):
    """Returns (total_bytes, [offset of d_s, d_x, d_dt, d_A, d_B, d_C, d_D])."""
    offs = (ctypes.c_size_t * 7)()
    total = load().ssm_scan_dgrad_layout(ctypes.byref(desc), ctypes.byref(offs))
    return total, list(offs)


def ssm_scan_workspace_bytes(desc: SsmScanDesc, backward: int) -> int:
    return load().ssm_scan_workspace_bytes(ctypes.byref(desc), int(backward))


def ssm_conv_fwd(sx, w, out, n_s, n_t, d_inner, d_conv, io_dtype, apply_silu, stream=None):
    rc = load().ssm_conv_fwd(_ptr(sx), _ptr(w), _ptr(out), int(n_s), int(n_t), int(d_inner),
                             int(d_conv), int(io_dtype), int(apply_silu), _stream(stream))
    return _check(rc, "ssm_conv_fwd")


def ssm_conv_bwd_workspace_bytes(n_s, n_t, d_inner, d_conv) -> int:
    return load().ssm_conv_bwd_workspace_bytes(int(n_s), int(n_t), int(d_inner), int(d_conv))


def ssm_conv_bwd(sx, w, dout, dgrad, n_s, n_t, d_inner, d_conv, io_dtype, apply_silu, workspace,
                 workspace_bytes, stream=None):
    rc = load().ssm_conv_bwd(_ptr(sx), _ptr(w), _ptr(dout), _ptr(dgrad), int(n_s), int(n_t),
                             int(d_inner), int(d_conv), int(io_dtype), int(apply_silu),
                             _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check(rc, "ssm_conv_bwd")


def selective_scan_fwd(desc, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                       conv_state_out, workspace, workspace_bytes, stream=None):
    rc = load().selective_scan_fwd(ctypes.byref(desc), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(conv_w),
                                   _ptr(conv_state), _ptr(out), _ptr(conv_state_out),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check(rc, "selective_scan_fwd")


def selective_scan_fwd_static(desc, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                              conv_state_out, err=None, stream=None):
    rc = load().selective_scan_fwd_static(ctypes.byref(desc), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                                          _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(conv_w),
                                          _ptr(conv_state), _ptr(out), _ptr(conv_state_out),
                                          _ptr(err), _stream(stream))
    return _check(rc, "selective_scan_fwd_static")


def make_ext(dt_bias=None, z=None, cu_seqlens=None, total_tokens=0) -> SsmScanExt:
    return SsmScanExt(_ptr(dt_bias), _ptr(z), _ptr(cu_seqlens), int(total_tokens))


def ssm_scan_ext_out_bytes(desc: SsmScanDesc, ext: Optional[SsmScanExt]):
    """(total bytes, state block offset); (0, 0) if invalid."""
    off = ctypes.c_size_t(0)
    n = load().ssm_scan_ext_out_bytes(ctypes.byref(desc), None if ext is None else ctypes.byref(ext),
                                      ctypes.byref(off))
    return int(n), int(off.value)


def ssm_scan_fwd_plan(desc: SsmScanDesc, ext: Optional[SsmScanExt] = None) -> Optional[str]:
    """The forward's kernel family for this descriptor (None if invalid)."""
    r = load().ssm_scan_fwd_plan(ctypes.byref(desc), None if ext is None else ctypes.byref(ext))
    return None if r is None else r.decode()


def selective_scan_fwd_ext(desc, ext, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                           conv_state_out, workspace, workspace_bytes, stream=None):
    rc = load().selective_scan_fwd_ext(ctypes.byref(desc), None if ext is None else ctypes.byref(ext),
                                       _ptr(s), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(D), _ptr(ids), _ptr(conv_w), _ptr(conv_state),
                                       _ptr(out), _ptr(conv_state_out), _ptr(workspace),
                                       int(workspace_bytes), _stream(stream))
    return _check(rc, "selective_scan_fwd_ext")


def selective_scan_bwd(desc, s, x, dt, A, B, C, D, ids, dout, dgrad, workspace,
                       workspace_bytes, stream=None):
    rc = load().selective_scan_bwd(ctypes.byref(desc), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(dout),
                                   _ptr(dgrad), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream))
    return _check(rc, "selective_scan_bwd")


def selective_scan_bwd_conv(desc, s, x, dt, A, B, C, D, ids, conv_w, conv_state, dout, dgrad,
                            workspace, workspace_bytes, stream=None):
    rc = load().selective_scan_bwd_conv(ctypes.byref(desc), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                                        _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(conv_w),
                                        _ptr(conv_state), _ptr(dout), _ptr(dgrad), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream))
    return _check(rc, "selective_scan_bwd_conv")


def selective_state_update(desc, s, x, dt, dt_bias, A, B, C, D, z, ids, conv_w, conv_state, y,
                           err, stream=None):
    rc = load().selective_state_update(ctypes.byref(desc), _ptr(s), _ptr(x), _ptr(dt),
                                       _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                       _ptr(ids), _ptr(conv_w), _ptr(conv_state), _ptr(y),
                                       _ptr(err), _stream(stream))
    return _check(rc, "selective_state_update")


def ssm_get_device_error(workspace, stream=None) -> int:
    bits = ctypes.c_uint32(0)
    _check(load().ssm_get_device_error(_ptr(workspace), _stream(stream), ctypes.byref(bits)),
           "ssm_get_device_error")
    return bits.value
