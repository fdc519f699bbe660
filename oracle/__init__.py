"""Float64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports or calls it, and it shares no code
with that path.

The arithmetic lives in ``ssm_oracle.c`` (plain sequential C in float64,
rows split over threads by head).  This module converts numpy inputs to
float64, applies the head-to-group map and calls it.

Where the pages leave a step open this oracle takes these readings:
  * head h reads B/C group ``h // (n_head // n_group)`` (contiguous heads
    share a group); the ggmlR ssm_scan contract only fixes the group axis;
  * ``ids[i]`` selects the state row sequence i starts from; its final
    state is written to row i of the state block (sequence order);
  * dt is used as given; ``dt_softplus`` applies softplus with the
    threshold-20 form of "mambazip mamba1/model.rs" (softplus);
  * with the fused conv, D multiplies the scan input u = SiLU(conv(x));
  * ``scan_fwd_ext``: the dt bias is added to the raw dt before softplus and
    the gate multiplies the whole y (C.h + D.u) by SiLU(z), as the decode step
    of "mambazip mamba1/model.rs" (forward_impl) does per token; sequences
    packed on one token axis (the RWKV-6/7 shapes of "ggmlR
    tests/testthat/test-ssm-rwkv.R", equal lengths there) may have different lengths, given as offsets cu_seqlens, and each
    starts from its own state and conv-state row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libssm_oracle.so")
_lock = threading.Lock()
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
                ("n_head", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("n_group", ctypes.c_int64),
                ("n_state_rows", ctypes.c_int64), ("a_per_state", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("has_D", ctypes.c_int32),
                ("dt_softplus", ctypes.c_int32)]


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c with gcc (no fast-math, no FP contraction)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("SSM_ORACLE_LIB")  # a planted-mistake build, in tests only
            if not path:
                if not os.path.exists(_LIB_PATH) or \
                        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                    build()
                path = _LIB_PATH
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            lib.oracle_scan_fwd.argtypes = [ctypes.POINTER(_Dims), P] + [P] * 13 + [ctypes.c_int]
            lib.oracle_scan_fwd.restype = ctypes.c_int
            lib.oracle_scan_bwd.argtypes = [ctypes.POINTER(_Dims), P] + [P] * 21 + [ctypes.c_int]
            lib.oracle_scan_bwd.restype = ctypes.c_int
            lib.oracle_conv_fwd.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
            lib.oracle_conv_fwd.restype = ctypes.c_int
            lib.oracle_conv_bwd.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
            lib.oracle_conv_bwd.restype = ctypes.c_int
            lib.oracle_state_update.argtypes = [ctypes.POINTER(_Dims), P] + [P] * 13
            lib.oracle_state_update.restype = ctypes.c_int
            lib.oracle_threads_used.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int]
            lib.oracle_threads_used.restype = ctypes.c_int
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    # never more than the 16 host threads a GPU machine grants one card
    return max(1, min(n, 16))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def group_of_head(n_head: int, n_group: int) -> np.ndarray:
    if n_head % n_group:
        raise ValueError("n_head must be a multiple of n_group")
    return (np.arange(n_head, dtype=np.int64) // (n_head // n_group)).astype(np.int64)


def _dims(n_seqs, n_tokens, n_head, head_dim, d_state, n_group, n_state_rows,
          a_per_state, d_conv, has_D, dt_softplus) -> _Dims:
    return _Dims(int(n_seqs), int(n_tokens), int(n_head), int(head_dim), int(d_state),
                 int(n_group), int(n_state_rows), int(bool(a_per_state)), int(d_conv),
                 int(bool(has_D)), int(bool(dt_softplus)))


def scan_fwd(s, x, dt, A, B, C, D, ids, *, conv_w=None, conv_state=None,
             dt_softplus=False, grp_of_head=None, n_threads: Optional[int] = None):
    """Sequential f64 selective scan.

    Shapes (row-major): s [R][H][P][N]; x [S][L][H][P]; dt [S][L][H];
    A [H][N] or [H]; B, C [S][L][G][N]; D [H] or None; ids [S];
    conv_w [H][K] (fused causal conv + SiLU, head_dim 1) or None;
    conv_state [R][H][K-1] or None (zeros).

    Returns (y [S][L][H][P], state [S][H][P][N], conv_state_out [S][H][K-1] or None).
    """
    s, x, dt, A, B, C, D = map(_f64, (s, x, dt, A, B, C, D))
    conv_w, conv_state = _f64(conv_w), _f64(conv_state)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    S, L, H, P = x.shape
    R, N = s.shape[0], s.shape[3]
    G = B.shape[2]
    K = 0 if conv_w is None else conv_w.shape[1]
    grp = group_of_head(H, G) if grp_of_head is None else np.ascontiguousarray(grp_of_head, np.int64)
    d = _dims(S, L, H, P, N, G, R, A.ndim == 2, K, D is not None, dt_softplus)
    y = np.zeros((S, L, H, P))
    st = np.zeros((S, H, P, N))
    cso = np.zeros((S, H, max(K - 1, 0))) if K else None
    lib = _load()
    rc = lib.oracle_scan_fwd(ctypes.byref(d), _ptr(grp), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                             _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(conv_w),
                             _ptr(conv_state), _ptr(y), _ptr(st), _ptr(cso),
                             n_threads or default_threads())
    if rc:
        raise ValueError(f"oracle_scan_fwd failed ({rc})")
    return y, st, cso


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def scan_fwd_ext(s, x, dt, A, B, C, D, ids, *, cu_seqlens=None, dt_bias=None, z=None,
                 conv_w=None, conv_state=None, dt_softplus=False, grp_of_head=None,
                 n_threads: Optional[int] = None):
    """``scan_fwd`` with the extras of the per-token step of "mambazip
    mamba1/model.rs" (forward_impl): dt = dt_raw + dt_bias before softplus, and
    y = (C.h + D.u) * SiLU(z); and with sequences packed on one token axis (the
    RWKV-6/7 shapes of "ggmlR tests/testthat/test-ssm-rwkv.R" start a fresh
    state at every sequence), sequence i
    being tokens cu_seqlens[i] .. cu_seqlens[i+1]-1.

    Without cu_seqlens the shapes are those of ``scan_fwd``.  With it: x and z
    [T][H][P], dt [T][H], B and C [T][G][N], and y comes back as [T][H][P];
    each sequence is ``scan_fwd`` over its own tokens from state row ids[i]
    (conv-state row ids[i]).  dt_bias [H] or None; z like x or None.

    Returns (y, state [S][H][P][N], conv_state_out [S][H][K-1] or None).
    """
    dt = _f64(dt)
    if dt_bias is not None:
        dt = dt + _f64(dt_bias)  # broadcast over the head axis, the last one of dt
    kw = dict(conv_w=conv_w, conv_state=conv_state, dt_softplus=dt_softplus,
              grp_of_head=grp_of_head, n_threads=n_threads)
    if cu_seqlens is None:
        y, st, cso = scan_fwd(s, x, dt, A, B, C, D, ids, **kw)
    else:
        x, B, C = _f64(x), _f64(B), _f64(C)
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        n_seqs = len(cu) - 1
        H, P, N = x.shape[1], x.shape[2], np.asarray(s).shape[3]
        K = 0 if conv_w is None else np.asarray(conv_w).shape[1]
        y = np.zeros(x.shape)
        st = np.zeros((n_seqs, H, P, N))
        cso = np.zeros((n_seqs, H, max(K - 1, 0))) if K else None
        for i in range(n_seqs):
            a, b = int(cu[i]), int(cu[i + 1])
            yi, si, ci = scan_fwd(s, x[None, a:b], dt[None, a:b], A, B[None, a:b], C[None, a:b], D,
                                  np.asarray(ids)[i:i + 1], **kw)
            y[a:b] = yi[0]
            st[i] = si[0]
            if K:
                cso[i] = ci[0]
    if z is not None:
        y = y * _silu(_f64(z))
    return y, st, cso


def scan_bwd(s, x, dt, A, B, C, D, ids, dy, dstate, *, conv_w=None, conv_state=None,
             dt_softplus=False, grp_of_head=None, n_threads: Optional[int] = None):
    """Reverse-time adjoint of ``scan_fwd``.

    Returns a dict with d_s, d_x, d_dt, d_A, d_B, d_C and d_D (None without D);
    with the fused conv (conv_w [H][K], head_dim 1; conv_state [R][H][K-1] or
    None for zeros) d_x is the gradient of the pre-conv input and the dict
    also holds d_conv_w [H][K] and d_conv_state [R][H][K-1].
    """
    s, x, dt, A, B, C, D, dy, dstate = map(_f64, (s, x, dt, A, B, C, D, dy, dstate))
    conv_w, conv_state = _f64(conv_w), _f64(conv_state)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    S, L, H, P = x.shape
    R, N = s.shape[0], s.shape[3]
    G = B.shape[2]
    K = 0 if conv_w is None else conv_w.shape[1]
    grp = group_of_head(H, G) if grp_of_head is None else np.ascontiguousarray(grp_of_head, np.int64)
    d = _dims(S, L, H, P, N, G, R, A.ndim == 2, K, D is not None, dt_softplus)
    out = dict(d_s=np.zeros_like(s), d_x=np.zeros_like(x), d_dt=np.zeros_like(dt),
               d_A=np.zeros_like(A), d_B=np.zeros_like(B), d_C=np.zeros_like(C),
               d_D=None if D is None else np.zeros_like(D),
               d_conv_w=np.zeros((H, K)) if K else None,
               d_conv_state=np.zeros((R, H, K - 1)) if K else None)
    lib = _load()
    rc = lib.oracle_scan_bwd(ctypes.byref(d), _ptr(grp), _ptr(s), _ptr(x), _ptr(dt), _ptr(A),
                             _ptr(B), _ptr(C), _ptr(D), _ptr(ids), _ptr(conv_w), _ptr(conv_state),
                             _ptr(dy), _ptr(dstate),
                             _ptr(out["d_s"]), _ptr(out["d_x"]), _ptr(out["d_dt"]),
                             _ptr(out["d_A"]), _ptr(out["d_B"]), _ptr(out["d_C"]),
                             _ptr(out["d_D"]), _ptr(out["d_conv_w"]), _ptr(out["d_conv_state"]),
                             n_threads or default_threads())
    if rc:
        raise ValueError(f"oracle_scan_bwd failed ({rc})")
    return out


def conv_fwd(sx, w, apply_silu=False):
    """ggml ssm_conv: sx [n_s][d_inner][d_conv-1+n_t], w [d_inner][d_conv]
    -> out [n_s][n_t][d_inner]."""
    sx, w = _f64(sx), _f64(w)
    n_s, d_inner, length = sx.shape
    K = w.shape[1]
    n_t = length - (K - 1)
    if n_t < 0 or w.shape[0] != d_inner:
        raise ValueError("bad conv shapes")
    out = np.zeros((n_s, n_t, d_inner))
    rc = _load().oracle_conv_fwd(_ptr(sx), _ptr(w), _ptr(out), n_s, n_t, d_inner, K,
                                 int(bool(apply_silu)))
    if rc:
        raise ValueError(f"oracle_conv_fwd failed ({rc})")
    return out


def conv_bwd(sx, w, dout, apply_silu=False):
    """Backward of ``conv_fwd`` (the ggmlR ssm_conv backward): sx [n_s][d_inner]
    [d_conv-1+n_t], w [d_inner][d_conv], dout [n_s][n_t][d_inner] ->
    (d_sx with the shape of sx, d_w with the shape of w)."""
    sx, w, dout = _f64(sx), _f64(w), _f64(dout)
    n_s, d_inner, length = sx.shape
    K = w.shape[1]
    n_t = length - (K - 1)
    if n_t < 0 or w.shape[0] != d_inner or dout.shape != (n_s, n_t, d_inner):
        raise ValueError("bad conv shapes")
    d_sx = np.zeros_like(sx)
    d_w = np.zeros_like(w)
    rc = _load().oracle_conv_bwd(_ptr(sx), _ptr(w), _ptr(dout), _ptr(d_sx), _ptr(d_w), n_s, n_t,
                                 d_inner, K, int(bool(apply_silu)))
    if rc:
        raise ValueError(f"oracle_conv_bwd failed ({rc})")
    return d_sx, d_w


def state_update(s, x, dt, A, B, C, D, ids, *, dt_bias=None, z=None, conv_w=None,
                 conv_state=None, dt_softplus=False, grp_of_head=None):
    """One decode token of every sequence ("mambazip mamba1/model.rs",
    forward_impl's single-token step).

    Shapes (row-major): s [R][H][P][N]; x [S][H][P]; dt [S][H]; A [H][N] or [H];
    B, C [S][G][N]; D [H] or None; ids [S]; dt_bias [H] or None; z [S][H][P]
    or None; conv_w [H][K] with conv_state [R][H][K-1] (head_dim 1) or None.

    Returns (y [S][H][P], new s, new conv_state or None); the inputs are not
    modified.
    """
    s, x, dt, A, B, C, D = map(_f64, (s, x, dt, A, B, C, D))
    dt_bias, z, conv_w, conv_state = map(_f64, (dt_bias, z, conv_w, conv_state))
    s = s.copy()
    conv_state = None if conv_state is None else conv_state.copy()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    S, H, P = x.shape
    R, N = s.shape[0], s.shape[3]
    G = B.shape[1]
    K = 0 if conv_w is None else conv_w.shape[1]
    if K and conv_state is None:
        raise ValueError("the decode conv needs a conv state")
    grp = group_of_head(H, G) if grp_of_head is None else np.ascontiguousarray(grp_of_head, np.int64)
    d = _dims(S, 1, H, P, N, G, R, A.ndim == 2, K, D is not None, dt_softplus)
    y = np.zeros((S, H, P))
    rc = _load().oracle_state_update(ctypes.byref(d), _ptr(grp), _ptr(s), _ptr(x), _ptr(dt),
                                     _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                     _ptr(ids), _ptr(conv_w), _ptr(conv_state), _ptr(y))
    if rc:
        raise ValueError(f"oracle_state_update failed ({rc})")
    return y, s, conv_state


def threads_used(n_head: int, n_threads: Optional[int] = None) -> int:
    d = _dims(1, 1, n_head, 1, 1, 1, 1, 1, 0, 0, 0)
    return _load().oracle_threads_used(ctypes.byref(d), n_threads or default_threads())


def problem_fwd(prob, n_threads=None):
    """Oracle forward of a ssm_inputs.ScanProblem (its stored values)."""
    v = prob.value
    return scan_fwd(v("s"), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), prob.ids,
                    conv_w=v("conv_w") if prob.d_conv else None,
                    conv_state=v("conv_state") if prob.d_conv else None,
                    dt_softplus=prob.dt_softplus, n_threads=n_threads)


def problem_bwd(prob, n_threads=None):
    v = prob.value
    return scan_bwd(v("s"), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), prob.ids,
                    v("dy"), v("dstate"), conv_w=v("conv_w") if prob.d_conv else None,
                    conv_state=v("conv_state") if prob.d_conv else None,
                    dt_softplus=prob.dt_softplus, n_threads=n_threads)
