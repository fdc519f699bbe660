"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and rounds them to the stored dtypes.
It holds none of the scan's arithmetic and imports neither the oracle nor
the HIP library; both sides consume exactly the arrays it returns.

Every tensor is filled in blocks of 2**20 elements; block b of a tensor
draws from its own stream, ``numpy.random.default_rng`` (PCG64) seeded with
``[seed, tensor_index, b]``, so the values do not depend on how many threads
fill the blocks.  Values are drawn in float64
and rounded to float32 with round-to-nearest-even (numpy's cast); tensors
stored as bfloat16 are then rounded from that float32 to bfloat16, again
round-to-nearest-even.  ``N(mu, sigma)`` below takes sigma as the standard
deviation.

Operand layouts are row-major, slowest axis first, and follow the ggml
``ssm_scan`` tensor contract (ggmlR test-ssm-rwkv.R, "make_scan"), whose
``ne`` lists are fastest-first:

    s      [n_state_rows][n_head][head_dim][d_state]   float32
    x      [n_seqs][n_tokens][n_head][head_dim]         io dtype
    dt     [n_seqs][n_tokens][n_head]                   io dtype
    A      [n_head][d_state] (Mamba-1) or [n_head]      float32
    B, C   [n_seqs][n_tokens][n_group][d_state]         io dtype
    D      [n_head]                                     float32
    ids    [n_seqs]                                     int32
    conv_w [n_head][d_conv]                             float32 (Mamba-1 only)

For the Mamba-1 form ``head_dim == 1`` and ``n_head == d_inner``.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# Fixed stream index per tensor, so adding a tensor never shifts another's values.
_STREAM = {
    "x": 1, "dt": 2, "A": 3, "B": 4, "C": 5, "D": 6, "conv_w": 7, "s": 8,
    "ids": 9, "conv_state": 10, "dy": 11, "dstate": 12, "sx": 13, "probe": 14, "dout": 15,
    "dt_bias": 16, "z": 17, "lengths": 18,
}


_BLOCK = 1 << 20  # elements per independently seeded block
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures as cf
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:
            n = os.cpu_count() or 1
        _POOL = cf.ThreadPoolExecutor(max_workers=max(1, min(n, 16)))
    return _POOL


def _rng(seed: int, name: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAM[name], int(block)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), as uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of each bfloat16 bit pattern."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Stored:
    """One tensor as stored: ``bits`` holds what goes to the device (float32,
    or uint16 bfloat16 bits), ``value`` its exact float32 value."""
    bits: np.ndarray
    value: np.ndarray
    dtype: str  # "f32" or "bf16"


def _draw(seed: int, name: str, shape, dtype: str, fn) -> Stored:
    """Fill a tensor block by block; block b draws ``fn(rng_b, n)`` float64
    values from its own stream [seed, tensor, b] and rounds them to ``dtype``."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    total = int(np.prod(shape)) if len(shape) else 1
    value = np.empty(total, dtype=np.float32)
    bits = value if dtype == "f32" else np.empty(total, dtype=np.uint16)

    def work(b):
        lo = b * _BLOCK
        hi = min(total, lo + _BLOCK)
        v32 = np.asarray(fn(_rng(seed, name, b), hi - lo), dtype=np.float64).astype(np.float32)
        if dtype == "f32":
            value[lo:hi] = v32
        else:
            bb = f32_to_bf16_bits(v32)
            bits[lo:hi] = bb
            value[lo:hi] = bf16_bits_to_f32(bb)

    nblk = (total + _BLOCK - 1) // _BLOCK
    if nblk <= 1:
        for b in range(nblk):
            work(b)
    else:
        list(_pool().map(work, range(nblk)))
    return Stored(bits.reshape(shape), value.reshape(shape), dtype)


def _const(v64, dtype: str = "f32") -> Stored:
    """A tensor whose values are given (rounded to ``dtype``), not drawn."""
    v32 = np.ascontiguousarray(np.asarray(v64, dtype=np.float64), dtype=np.float32)
    if dtype == "f32":
        return Stored(v32, v32, "f32")
    bb = f32_to_bf16_bits(v32)
    return Stored(bb, bf16_bits_to_f32(bb), "bf16")


def _uniform(lo, hi):
    return lambda rng, n: rng.uniform(lo, hi, size=n)


def _normal(std):
    return lambda rng, n: rng.standard_normal(size=n) * std


def _softplus_of_normal(shift):
    # Input recipe only: dt is drawn as softplus(N(0,1) + shift), i.e. already
    # positive, and handed to the scan as given.
    def f(rng, n):
        z = rng.standard_normal(size=n) + shift
        return np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))
    return f


@dataclass
class ScanProblem:
    """Operands of one selective-scan call plus its dimensions."""
    n_seqs: int
    n_tokens: int
    n_head: int
    head_dim: int
    d_state: int
    n_group: int
    n_state_rows: int
    a_per_state: bool
    d_conv: int
    io: str
    has_D: bool
    dt_softplus: bool
    chunk: int
    t: Dict[str, Stored] = field(default_factory=dict)
    ids: Optional[np.ndarray] = None

    @property
    def d_inner(self) -> int:
        return self.n_head * self.head_dim

    def value(self, name: str) -> Optional[np.ndarray]:
        s = self.t.get(name)
        return None if s is None else s.value


def make_problem(*, n_seqs, n_tokens, n_head, d_state, head_dim=1, n_group=1,
                 a_per_state=True, d_conv=4, io="f32", seed=0,
                 h0_std=0.0, n_state_rows=None, ids="identity",
                 A_kind="s4d", A_range=(1.0, 16.0), bc_std=1.0,
                 dt_shift=-2.0, x_range=1.0, has_D=True, conv_state_std=None,
                 dt_softplus=False, chunk=0, with_dout=False, dstate_std=0.0,
                 dy_std=1.0) -> ScanProblem:
    """Draw one seeded problem.

    A_kind: "s4d" gives A[h][n] = -exp(log(n+1)) (the same row for every
    channel; needs a_per_state), "uniform" gives -U(A_range) per entry.
    ids: "identity" (ids[i] = i), "perm" (a seeded permutation of
    0..n_state_rows-1, first n_seqs entries), or an explicit int array.
    """
    if n_state_rows is None:
        n_state_rows = n_seqs
    P, H, N, G, L = head_dim, n_head, d_state, n_group, n_tokens
    prob = ScanProblem(n_seqs, L, H, P, N, G, n_state_rows, bool(a_per_state),
                       int(d_conv), io, bool(has_D), bool(dt_softplus), int(chunk))
    t = prob.t
    t["x"] = _draw(seed, "x", (n_seqs, L, H, P), io, _uniform(-x_range, x_range))
    t["dt"] = _draw(seed, "dt", (n_seqs, L, H), io, _softplus_of_normal(dt_shift))
    a_shape = (H, N) if a_per_state else (H,)
    if A_kind == "s4d":
        if not a_per_state:
            raise ValueError("s4d A needs a per-state A")
        row = -np.exp(np.log(np.arange(1, N + 1, dtype=np.float64)))
        t["A"] = _const(np.broadcast_to(row, (H, N)))
    elif A_kind == "uniform":
        t["A"] = _draw(seed, "A", a_shape, "f32", lambda rng, n: -rng.uniform(*A_range, size=n))
    else:
        raise ValueError(A_kind)
    t["B"] = _draw(seed, "B", (n_seqs, L, G, N), io, _normal(bc_std))
    t["C"] = _draw(seed, "C", (n_seqs, L, G, N), io, _normal(bc_std))
    if has_D:
        t["D"] = _draw(seed, "D", (H,), "f32", _normal(1.0))
    if d_conv:
        if P != 1:
            raise ValueError("the fused conv is defined for the Mamba-1 form (head_dim 1)")
        t["conv_w"] = _draw(seed, "conv_w", (H, d_conv), "f32", _uniform(-0.5, 0.5))
        if conv_state_std:
            t["conv_state"] = _draw(seed, "conv_state", (n_state_rows, H, d_conv - 1), "f32",
                                    _normal(conv_state_std))
    s_shape = (n_state_rows, H, P, N)
    if h0_std:
        t["s"] = _draw(seed, "s", s_shape, "f32", _normal(h0_std))
    else:
        t["s"] = _const(np.zeros(s_shape))
    if isinstance(ids, str):
        if ids == "identity":
            if n_seqs > n_state_rows:
                raise ValueError("identity ids need n_state_rows >= n_seqs")
            idv = np.arange(n_seqs, dtype=np.int32)
        elif ids == "perm":
            idv = _rng(seed, "ids").permutation(n_state_rows)[:n_seqs].astype(np.int32)
        else:
            raise ValueError(ids)
    else:
        idv = np.ascontiguousarray(ids, dtype=np.int32)
    prob.ids = idv
    if with_dout:
        add_dout(prob, seed, dy_std=dy_std, dstate_std=dstate_std)
    return prob


def add_dout(prob: ScanProblem, seed: int, dy_std=1.0, dstate_std=0.0) -> None:
    """Upstream gradient, packed like the forward result: dy then dstate."""
    shape_y = (prob.n_seqs, prob.n_tokens, prob.n_head, prob.head_dim)
    prob.t["dy"] = _draw(seed, "dy", shape_y, prob.io, _normal(dy_std))
    shape_s = (prob.n_seqs, prob.n_head, prob.head_dim, prob.d_state)
    if dstate_std:
        prob.t["dstate"] = _draw(seed, "dstate", shape_s, "f32", _normal(dstate_std))
    else:
        prob.t["dstate"] = _const(np.zeros(shape_s))


# The workloads measured and parity-tested.  Shapes and distributions are the
# ones the benchmark configurations state; where they leave a choice open the
# choice is noted beside it.
def config(name: str) -> ScanProblem:
    if name == "C0":   # tiny Mamba-1, fp32, fused conv, h0 = 0
        return make_problem(n_seqs=1, n_tokens=64, n_head=32, d_state=16, d_conv=4,
                            io="f32", seed=0xC0)
    if name == "C1":   # Mamba-1 small-model shape, fp32, h0 ~ N(0, 0.1)
        return make_problem(n_seqs=8, n_tokens=2048, n_head=512, d_state=16, d_conv=4,
                            io="f32", seed=0xC1, h0_std=0.1)
    if name == "C2":   # Mamba-1 large layer, bf16 x/dt/B/C/y, fp32 state/A/D, h0 = 0
        return make_problem(n_seqs=8, n_tokens=4096, n_head=5120, d_state=16, d_conv=4,
                            io="bf16", seed=0xC2)
    if name == "C3":   # Mamba-2 form; x, h0 and D are not stated: U(-1,1), N(0,0.1), N(0,1)
        return make_problem(n_seqs=4, n_tokens=4096, n_head=80, head_dim=64, d_state=128,
                            n_group=1, a_per_state=False, d_conv=0, io="bf16", seed=0xC3,
                            h0_std=0.1, ids="perm", A_kind="uniform", A_range=(1.0, 16.0),
                            bc_std=1.0 / np.sqrt(128.0), chunk=256)
    if name == "C4":   # backward of the C2 scan (no conv): C2's draws, dy ~ N(0,1), dstate = 0
        p = make_problem(n_seqs=8, n_tokens=4096, n_head=5120, d_state=16, d_conv=0,
                         io="bf16", seed=0xC2)
        add_dout(p, 0xC4)
        return p
    if name == "C10":  # backward of the whole C2 layer (conv + SiLU + scan): C2's draws, dy ~ N(0,1)
        p = config("C2")
        add_dout(p, 0xCA)
        return p
    if name == "C8":   # backward of the C3 Mamba-2 scan: C3's draws, dy ~ N(0,1), dstate = 0
        p = config("C3")
        add_dout(p, 0xC8)
        return p
    raise KeyError(name)


CONFIG_NAMES = ("C0", "C1", "C2", "C3", "C4")


class ConvProblem:
    """Inputs of the standalone conv backward (ssm_conv_bwd): sx
    [n_s][d_inner][d_conv-1+n_t] (io dtype), w [d_inner][d_conv] (f32) and
    the upstream gradient dout [n_s][n_t][d_inner] (f32)."""

    def __init__(self, n_s, n_t, d_inner, d_conv, io, apply_silu, seed):
        self.n_s, self.n_t, self.d_inner, self.d_conv = n_s, n_t, d_inner, d_conv
        self.io, self.apply_silu, self.seed = io, apply_silu, seed
        self.sx = _draw(seed, "sx", (n_s, d_inner, d_conv - 1 + n_t), io, _uniform(-1.0, 1.0))
        self.w = _draw(seed, "conv_w", (d_inner, d_conv), "f32", _uniform(-0.5, 0.5))
        self.dout = _draw(seed, "dout", (n_s, n_t, d_inner), "f32", _normal(1.0))


def conv_config(name: str) -> ConvProblem:
    if name == "C5":   # conv + SiLU backward of the C2 activations: 8 x 4096 x 5120, d_conv 4
        return ConvProblem(8, 4096, 5120, 4, "bf16", True, 0xC5)
    if name == "C11":  # the standalone conv + SiLU forward of the same activations (dout unused)
        return ConvProblem(8, 4096, 5120, 4, "bf16", True, 0xCB)
    raise KeyError(name)


def make_decode_problem(*, with_z=False, dt_bias_range=None, **kw) -> ScanProblem:
    """Operands of one decode step (selective_state_update): a one-token
    problem of ``make_problem`` (x [S][1][H][P] is laid out as [S][H][P], B and
    C as [S][G][N], dt as [S][H]), plus z ~ N(0,1) in the io dtype when
    with_z, and dt_bias ~ U(dt_bias_range) per head when given."""
    kw.setdefault("n_tokens", 1)
    if kw["n_tokens"] != 1:
        raise ValueError("a decode step has one token")
    p = make_problem(**kw)
    S, H, P = p.n_seqs, p.n_head, p.head_dim
    seed = kw.get("seed", 0)
    if with_z:
        p.t["z"] = _draw(seed, "z", (S, H, P), p.io, _normal(1.0))
    if dt_bias_range is not None:
        p.t["dt_bias"] = _draw(seed, "dt_bias", (H,), "f32", _uniform(*dt_bias_range))
    return p


def make_varlen_problem(*, lengths, n_state_rows=None, ids="perm", with_z=False,
                        dt_bias_range=None, seed=0, **kw) -> ScanProblem:
    """Sequences of the given lengths packed on one token axis: one draw of
    ``make_problem`` with a single sequence of sum(lengths) tokens (its x
    [1][T][H][P] is the packed [T][H][P], and so on), n_seqs set to the
    number of lengths, n_tokens to the longest, cu_seqlens the offsets; plus
    z ~ N(0,1) in the io dtype when with_z and dt_bias ~ U(dt_bias_range)
    per head when given."""
    lengths = np.asarray(lengths, dtype=np.int64)
    S, T = len(lengths), int(lengths.sum())
    R = S if n_state_rows is None else n_state_rows
    if isinstance(ids, str):
        idv = (np.arange(S) if ids == "identity" else _rng(seed, "ids").permutation(R)[:S])
    else:
        idv = ids
    p = make_problem(n_seqs=1, n_tokens=T, n_state_rows=R, ids=np.asarray(idv, np.int32), seed=seed,
                     **kw)
    p.n_seqs, p.n_tokens = S, int(lengths.max()) if S else 0
    p.cu_seqlens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    p.total_tokens = T
    if with_z:
        p.t["z"] = _draw(seed, "z", (1, T, p.n_head, p.head_dim), p.io, _normal(1.0))
    if dt_bias_range is not None:
        p.t["dt_bias"] = _draw(seed, "dt_bias", (p.n_head,), "f32", _uniform(*dt_bias_range))
    return p


def length_mix(n_seqs: int, total: int, seed: int, lo=0.25, hi=1.75) -> np.ndarray:
    """n_seqs lengths summing to total: U(lo, hi) times the mean length, rounded
    (a seeded mix of short and long sequences, most not multiples of 64)."""
    w = _rng(seed, "lengths").uniform(lo, hi, n_seqs)
    L = np.floor(w / w.sum() * total).astype(np.int64)
    L[-1] += total - L.sum()
    return L


def varlen_config(name: str) -> ScanProblem:
    if name == "C9":   # the C2 layer as one packed batch: 8 sequences of a length mix summing to
        # 8 x 4096 tokens, 5120 channels, d_state 16, d_conv 4, bf16; dt bias, softplus, z gate
        lengths = length_mix(8, 8 * 4096, 0xC9)
        return make_varlen_problem(lengths=lengths, n_head=5120, d_state=16, d_conv=4, io="bf16",
                                   seed=0xC9, h0_std=0.1, conv_state_std=0.5, dt_softplus=True,
                                   with_z=True, dt_bias_range=(-3.0, -1.0))
    raise KeyError(name)


def decode_config(name: str) -> ScanProblem:
    if name == "C6":   # Mamba-1 decode at the large layer: 256 sequences x 5120 channels, d_state 16
        return make_decode_problem(n_seqs=256, n_head=5120, d_state=16, d_conv=4, io="bf16",
                                   seed=0xC6, h0_std=0.1, conv_state_std=0.5, n_state_rows=256,
                                   ids="perm", with_z=True)
    if name == "C7":   # Mamba-2 decode at the C3 layer: 64 sequences x 80 heads x 64, d_state 128
        return make_decode_problem(n_seqs=64, n_head=80, head_dim=64, d_state=128, n_group=1,
                                   a_per_state=False, d_conv=0, io="bf16", seed=0xC7, h0_std=0.1,
                                   n_state_rows=64, ids="perm", A_kind="uniform",
                                   A_range=(1.0, 16.0), bc_std=1.0 / np.sqrt(128.0), with_z=True)
    raise KeyError(name)
