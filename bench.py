#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2]

One step is one selective_scan_fwd call (Mamba-1 form: gather of the initial
state by ids, causal depthwise conv + SiLU fused into the scan, the scan with
its output contraction, and the packed y | final-state write) on one batch
of seeded synthetic input of the named workload; --config C4 times the
reverse-time backward instead, C3 the Mamba-2 form.  Inputs are resident in
HBM before timing starts.  To keep the working set out of the 256 MB
last-level cache, steps rotate over enough copies of the inputs and outputs
that together exceed it.

Before any number is printed the first call's output is checked against the
float64 oracle (all elements for C0/C1, every token of sampled channels for
the larger workloads).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
# VALU peaks from the unit counts: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz =
# 39.3 T lane-instructions/s; the published 157.3 TFLOP/s fp32 vector figure
# counts an FMA as 2 flops and packed FP32 (two lanes' worth per instruction)
# on top, i.e. 78.6 T lane-FMA/s.  The kernels here use no packed FP32, so
# their issue ceiling is 39.3 T; both are reported.
VALU_PEAK_T = 78.6               # T lane-FMA/s with packed FP32 (the published figure)
VALU_ISSUE_T = 39.3              # T lane-instructions/s, one VALU op per lane per cycle
MFMA_BF16_PEAK_T = 2500.0        # dense bf16 MFMA, TFLOP/s
TRANS_COST = 4                   # v_exp_f32 / v_rcp_f32 against the packed peak (1/4 rate)
TRANS_ISSUE = 2                  # ... against the issue ceiling: measured at half the FMA rate
MALL_BYTES = 256 << 20
METRIC = "selective-scan effective HBM GB/s (% of peak) + channel-tokens/s, 1 GPU"

WORKLOADS = {
    "C0": "Mamba-1 fused conv+SiLU+scan forward, 1x64x32, d_state 16, d_conv 4, fp32",
    "C1": "Mamba-1 fused conv+SiLU+scan forward, 8x2048x512, d_state 16, d_conv 4, fp32",
    "C2": "Mamba-1 fused conv+SiLU+scan forward, 8x4096x5120, d_state 16, d_conv 4, "
          "bf16 x/dt/B/C/y, fp32 state/A/D",
    "C3": "Mamba-2 scan forward, 4x4096, 80 heads x 64, d_state 128, 1 group, bf16, "
          "fp32 state, permuted state ids",
    "C4": "Mamba-1 scan reverse-time backward of the 8x4096x5120 bf16 scan, fp32 grads",
    "C5": "ssm_conv backward (conv + SiLU) of the 8x4096x5120 bf16 activations, d_conv 4, "
          "fp32 gradients",
    "C6": "Mamba-1 single-token decode step of 256 sequences at the 5120-channel layer, "
          "d_state 16, d_conv 4, bf16 x/dt/B/C/z/y, fp32 states updated in place by permuted ids",
    "C7": "Mamba-2 single-token decode step of 64 sequences at the 80 heads x 64 layer, "
          "d_state 128, bf16 x/dt/B/C/z/y, fp32 states updated in place by permuted ids",
    "C8": "Mamba-2 scan reverse-time backward of the 4x4096, 80 heads x 64, d_state 128 bf16 scan, "
          "fp32 grads",
    "C10": "backward of the whole Mamba-1 layer (causal conv + SiLU + scan) at 8x4096x5120, d_state 16, "
           "d_conv 4, bf16 x/dt/B/C/dy, fp32 grads",
    "C11": "ssm_conv forward (causal depthwise conv + SiLU) of the 8x4096x5120 bf16 activations, d_conv 4",
    "C9": "Mamba-1 fused conv+SiLU+scan forward of 8 packed sequences of mixed lengths (32768 "
          "tokens) at the 5120-channel layer, d_state 16, d_conv 4, with dt bias + softplus and the "
          "SiLU(z) output gate, bf16 x/dt/B/C/z/y, fp32 state/A/D",
}


def algorithmic_bytes(p, backward=False) -> int:
    """Each input read once, each output written once (no re-reads, no workspace)."""
    io = 2 if p.io == "bf16" else 4
    S, L, H, P, N, G, R = p.n_seqs, p.n_tokens, p.n_head, p.head_dim, p.d_state, p.n_group, p.n_state_rows
    x = S * L * H * P * io
    dt = S * L * H * io
    bc = 2 * S * L * G * N * io
    a = (H * N if p.a_per_state else H) * 4
    d = H * 4 if p.has_D else 0
    w = H * p.d_conv * 4 if p.d_conv else 0
    state = S * H * P * N * 4
    ids = S * 4
    if not backward:
        y = S * L * H * P * io
        return x + dt + bc + a + d + w + state + ids + y + state
    dy = S * L * H * P * io
    grads = (R * H * P * N + S * L * H * P + S * L * H + (H * N if p.a_per_state else H) +
             2 * S * L * G * N + (H if p.has_D else 0)) * 4
    if p.d_conv:  # the conv weights in, their gradient and the conv-state rows' gradient out
        grads += (H * p.d_conv + R * H * (p.d_conv - 1)) * 4
    return x + dt + bc + a + d + w + state + ids + dy + state + grads


def valu_ops_per_channel_token(p, backward=False):
    """(VALU ops, transcendentals) the method needs per (sequence, channel,
    token); see valu_slots_per_channel_token for the count."""
    N = p.d_state
    if backward:
        ops, trans = 12 * N + 4, N
        if p.d_conv:
            ops, trans = ops + 3 * p.d_conv + 7, trans + 2
        return float(ops), float(trans)
    if p.a_per_state:
        ops, trans = 4 * N, N
    else:
        ops, trans = 3 * N + 1 / p.head_dim, 1 / p.head_dim
    ops += 2
    if p.d_conv:
        ops, trans = ops + p.d_conv + 3, trans + 2
    return float(ops), float(trans)


def issue_model(ops_trans, ch_tok, avg_s):
    """The same count against the non-packed issue ceiling (VALU_ISSUE_T, a
    transcendental taking TRANS_ISSUE slots)."""
    ops, trans = ops_trans
    slots = (ops + TRANS_ISSUE * trans) * ch_tok
    floor = slots / (VALU_ISSUE_T * 1e12)
    return {"peak": VALU_ISSUE_T, "unit": "T lane-instructions/s (no packed FP32)",
            "slots": int(slots), "floor_us": round(floor * 1e6, 2), "frac": round(floor / avg_s, 4)}


def valu_slots_per_channel_token(p, backward=False) -> float:
    """Issue slots the method needs per (sequence, channel, token), counting a
    transcendental (exp, reciprocal) as TRANS_COST slots.
    Forward, per state, Mamba-1 (A per state): decay exp(dt*A) (mul + exp),
    input term (mul), state update (fma), output term (fma).  Mamba-2 (A per
    head): input term, state update, output term; the decay is one mul + exp
    per (token, head), shared by the head's channels.  Per channel-token:
    dt*u (mul), D*u (fma); with the conv, its taps (fma each) and SiLU (mul,
    exp, add, rcp, mul).
    Backward (Mamba-1), per state: the recomputed decay and state (mul, exp,
    fma), the adjoint step (fma for C dy, mul for the decay), its products
    for du, ddt, dA, dB, dC (mul/fma each: 6), and the channel sums of dB
    and dC (add each); per channel-token: dt*u, du, ddt, dD (4)."""
    # with the fused conv the backward adds the recomputed conv and SiLU (K + 3
    # and 2 transcendentals), SiLU's derivative (4), the conv adjoint and the
    # weight gradient (2 K)
    ops, trans = valu_ops_per_channel_token(p, backward)
    return ops + TRANS_COST * trans


# HBM traffic of one call, from two rocprofv3 --pmc passes over
# "bench.py --config <C> --steps 3 --warmup 1 --no-cpu-baseline" (FETCH_SIZE, then
# WRITE_SIZE: KiB per dispatch, summed over the dispatches of one call), each scaled
# by COPY_FACTOR: the ratio of known bytes to what the same counter reads for a
# plain device copy of 1 GiB ("bench.py --copy-probe").  A figure holds only for the
# kernel sources it was taken on; bench.py reports null once any of them changes.
COPY_FACTOR = {"fetch": 1.99994, "write": 1.00000}
MEASURED_TRAFFIC = {
    "C1": {"sha256": "3faae9c4929597f0b48c263c0f643218feef324c205b8e93f4e5dc1260b16771", "fetch_kib": 34140.2, "write_kib": 33024.0},
    "C2": {"sha256": "3faae9c4929597f0b48c263c0f643218feef324c205b8e93f4e5dc1260b16771", "fetch_kib": 340956.4, "write_kib": 332296.0},
    "C3": {"sha256": "dfa33a9f4015ac56424fbdd57fb520ae911aa72b6a87607f9a9f96108eb09043", "fetch_kib": 143255.0, "write_kib": 174080.3},
    "C4": {"sha256": "2a46b022932ac6ec6fec633ef5221432a0374beec1c3222e02b0cf240b04e297", "fetch_kib": 1670396.2, "write_kib": 2964692.1},
    "C5": {"sha256": "19d21d3c16653649e1d9cac38de168171b782e33178b052b1b50c035b9a95dd5", "fetch_kib": 512932.3, "write_kib": 704850.3},
    "C6": {"sha256": "365057569e18c41ae6495048cfbeb33cacead190cc03a245029d5ac614a042b7", "fetch_kib": 52810.7, "write_kib": 99843.7},
    "C7": {"sha256": "365057569e18c41ae6495048cfbeb33cacead190cc03a245029d5ac614a042b7", "fetch_kib": 83410.5, "write_kib": 164502.2},
    "C8": {"sha256": "d400dd9f758bb898e47e5e8f43f2fb3cf32c2dab8cc83229deafe8dfe4da3fc5", "fetch_kib": 1351315.0, "write_kib": 2411816.2},
    "C9": {"sha256": "3c0e2ea0340a49be790cdacc592eb9c771e4a786aed94dd7657ca3a3703992e7", "fetch_kib": 506996.8, "write_kib": 330720.0},
    "C10": {"sha256": "2a46b022932ac6ec6fec633ef5221432a0374beec1c3222e02b0cf240b04e297", "fetch_kib": 1670588.0, "write_kib": 2966628.4},
    "C11": {"sha256": "4953558e4e65ac64e2be02ba4b598fe802356a85f0e8fe0be0a7f4cac01e0dea", "fetch_kib": 164316.8, "write_kib": 327680.0},
}
KERNEL_SOURCES = {
    "C0": ("scan_fwd.hip", "scan_fwd_ts.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C1": ("scan_fwd.hip", "scan_fwd_ts.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C2": ("scan_fwd.hip", "scan_fwd_ts.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C9": ("scan_fwd.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C3": ("scan_fwd.hip", "ssd_fwd.hip", "device_common.h"),
    "C4": ("scan_bwd.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C5": ("conv_bwd.hip", "device_common.h"),
    "C6": ("decode.hip", "device_common.h"),
    "C7": ("decode.hip", "device_common.h"),
    "C8": ("ssd_bwd.hip", "ssd_fwd.hip", "relay.h", "relay.hip", "device_common.h"),
    "C10": ("scan_bwd.hip", "scan_fwd_quad.hip", "relay.h", "relay.hip", "device_common.h"),
    "C11": ("conv_fwd.hip", "device_common.h"),
}


def kernel_sources_sha(name) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "selective_scan_recurrence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per call from the counter table above, or None when there is
    no figure for these sources."""
    m = MEASURED_TRAFFIC.get(name)
    if not m or None in COPY_FACTOR.values() or m["sha256"] != kernel_sources_sha(name):
        return None
    return int(round((m["fetch_kib"] * COPY_FACTOR["fetch"] + m["write_kib"] * COPY_FACTOR["write"]) * 1024))


def copy_probe(n_bytes=1 << 30, reps=3):
    """Plain device-to-device copies of n_bytes, for calibrating FETCH_SIZE and
    WRITE_SIZE: each dispatch reads and writes exactly n_bytes."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n_bytes, "reps": reps,
                      "ok": bool(torch.equal(dst[:1024], src[:1024]))}), flush=True)


SSD_Q = 64  # tokens per chunk of the chunked (MFMA) Mamba-2 path


def ssd_mfma_flops(p) -> int:
    """Dense-product flops of the chunked Mamba-2 form, per (sequence, head,
    64-token chunk): C B^T and M X on the causal triangle (Q(Q+1)/2 token
    pairs), the carried-state product C h^T and the state update X^T B."""
    q = SSD_Q
    chunks = -(-p.n_tokens // q)
    tri = q * (q + 1) // 2
    per = 2 * tri * p.d_state + 2 * tri * p.head_dim + 4 * q * p.d_state * p.head_dim
    return int(p.n_seqs * p.n_head * chunks * per)


def ssd_bwd_mfma_flops(p) -> int:
    """Dense-product flops of the chunked Mamba-2 backward, per (sequence, head,
    64-token chunk): S = C B^T and R = dY X^T on the causal tiles, M^T dY,
    Lm B and Lm^T C on the causal tiles, and the four Q x N x P products
    (B G^T, dY h_in, X G, the carry C^T dY), plus the recompute's state update."""
    q = SSD_Q
    chunks = -(-p.n_tokens // q)
    tri = q * (q + 1) // 2
    n, pd = p.d_state, p.head_dim
    per = 2 * tri * (n + pd) + 2 * tri * pd + 4 * tri * n + 5 * 2 * q * n * pd
    return int(p.n_seqs * p.n_head * chunks * per)


def uses_ssd(p) -> bool:
    return (not p.a_per_state and p.io == "bf16" and p.d_conv == 0 and p.head_dim in (32, 64)
            and p.d_state in (64, 128))


def _dev(stored, device):
    import torch
    bits = stored.bits
    if stored.dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(bits)).to(device)


def parity_gate(name, p, res):
    """Compares the first call's output with the oracle; raises on mismatch."""
    import torch
    import oracle
    rtol, atol = (1e-4, 1e-5) if p.io == "f32" else (2e-2, 1e-3)
    if name in ("C0", "C1"):
        y_o, st_o, _ = oracle.problem_fwd(p)
        ys, sts = res.y.double().cpu().numpy(), res.state.double().cpu().numpy()
        checked = y_o.size + st_o.size
    else:
        rng = np.random.default_rng(0xB0)
        heads = np.unique(np.concatenate([[0, p.n_head - 1], rng.choice(p.n_head, 8, replace=False)]))
        v = p.value
        grp = oracle.group_of_head(p.n_head, p.n_group)[heads]
        y_o, st_o, _ = oracle.scan_fwd(
            v("s")[:, heads], v("x")[:, :, heads], v("dt")[:, :, heads], v("A")[heads], v("B"),
            v("C"), v("D")[heads] if p.has_D else None, p.ids,
            conv_w=v("conv_w")[heads] if p.d_conv else None, grp_of_head=grp)
        hs = torch.as_tensor(heads, device=res.y.device)
        ys = res.y.index_select(2, hs).double().cpu().numpy()
        sts = res.state.index_select(1, hs).double().cpu().numpy()
        checked = y_o.size + st_o.size
    for got, want, what in ((ys, y_o, "y"), (sts, st_o, "state")):
        bad = ~(np.abs(got - want) <= atol + rtol * np.abs(want))
        if bad.any():
            raise SystemExit(f"parity gate failed on {name} {what}: {int(bad.sum())} elements "
                             f"outside rtol={rtol} atol={atol}")
    return {"checked_elements": int(checked), "rtol": rtol, "atol": atol,
            "max_abs_err_y": float(np.max(np.abs(ys - y_o)))}


def cpu_baseline(name, p, min_seconds=10.0, max_reps=50):
    """The float64 oracle, as it stands, on the host cores: the full workload
    for C0/C1, a bounded sample of channels for the larger ones, repeated
    until about min_seconds of CPU work have been timed (the rate is the
    mean over the repetitions)."""
    import oracle
    threads = oracle.default_threads()
    v = p.value
    if name in ("C0", "C1"):
        heads = np.arange(p.n_head)
        sample = "full workload"
    else:
        n = {"C2": 1024, "C4": 512, "C10": 512}.get(name, 8)
        heads = np.arange(n)
        sample = f"first {n} of {p.n_head} {'channels' if p.head_dim == 1 else 'heads'}, all sequences and tokens"
    args = (v("s")[:, heads], v("x")[:, :, heads], v("dt")[:, :, heads], v("A")[heads], v("B"),
            v("C"), v("D")[heads] if p.has_D else None, p.ids)
    grp = oracle.group_of_head(p.n_head, p.n_group)[heads]
    backward = name in ("C4", "C8", "C10")
    extra = (v("dy")[:, :, heads], v("dstate")[:, heads]) if backward else ()
    reps, sec = 0, 0.0
    while reps < max_reps and (reps == 0 or sec < min_seconds):
        t0 = time.perf_counter()
        if backward:
            oracle.scan_bwd(*args, *extra, conv_w=v("conv_w")[heads] if p.d_conv else None,
                            grp_of_head=grp, n_threads=threads)
        else:
            oracle.scan_fwd(*args, conv_w=v("conv_w")[heads] if p.d_conv else None, grp_of_head=grp,
                            n_threads=threads)
        sec += time.perf_counter() - t0
        reps += 1
    per = sec / reps
    frac = len(heads) / p.n_head
    gbs = algorithmic_bytes(p, backward) * frac / per / 1e9
    ch_tok = p.n_seqs * p.n_tokens * len(heads) * p.head_dim / per
    out = {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.threads_used(len(heads), threads),
           "kind": "oracle", "sample": f"{sample}; {reps} repetitions", "seconds": round(sec, 3),
           "channel_tokens_per_s": round(ch_tok, 1), "cpu": platform.processor() or platform.machine(),
           "nproc": os.cpu_count()}
    if name in ("C0", "C1"):  # the same workload on one thread
        t0 = time.perf_counter()
        oracle.scan_fwd(*args, conv_w=v("conv_w")[heads] if p.d_conv else None, grp_of_head=grp,
                        n_threads=1)
        one = time.perf_counter() - t0
        out["one_thread"] = {"value": round(algorithmic_bytes(p) / one / 1e9, 4), "unit": "GB/s",
                             "seconds": round(one, 3),
                             "channel_tokens_per_s": round(p.n_seqs * p.n_tokens * p.n_head / one, 1)}
    return out


def parity_gate_bwd(name, p, g):
    """Backward: every token of sampled channels (heads) against the oracle.
    Mamba-1 (fp32 arithmetic): per-element gradients with rtol 1e-4 and an
    absolute floor of 1e-5 x rms, channel and token sums with a floor of
    1e-4 x rms.  Mamba-2 (bf16 MFMA operands): rtol 2e-2 with a floor of
    1e-2 x rms for d_x and 2e-2 x rms for the sums (d_dt included)."""
    import torch
    import oracle
    rng = np.random.default_rng(0xB1)
    heads = np.unique(np.concatenate([[0, p.n_head - 1], rng.choice(p.n_head, 8, replace=False)]))
    v = p.value
    o = oracle.scan_bwd(v("s")[:, heads], v("x")[:, :, heads], v("dt")[:, :, heads], v("A")[heads],
                        v("B"), v("C"), v("D")[heads] if p.has_D else None, p.ids,
                        v("dy")[:, :, heads], v("dstate")[:, heads],
                        conv_w=v("conv_w")[heads] if p.d_conv else None,
                        grp_of_head=np.zeros(len(heads), np.int64))
    hs = torch.as_tensor(heads, device=g["d_x"].device)
    mfma = uses_ssd(p)
    rtol = 2e-2 if mfma else 1e-4
    fe, fs = (1e-2, 2e-2) if mfma else (1e-5, 1e-4)
    fdt = fs if mfma else fe  # Mamba-2: d_dt sums over the head's channels and states
    picks = {"d_x": (g["d_x"].index_select(2, hs), fe), "d_dt": (g["d_dt"].index_select(2, hs), fdt),
             "d_A": (g["d_A"].index_select(0, hs), fs), "d_s": (g["d_s"].index_select(1, hs), fs)}
    if p.has_D:
        picks["d_D"] = (g["d_D"].index_select(0, hs), fs)
    if p.d_conv:
        picks["d_conv_w"] = (g["d_conv_w"].index_select(0, hs), fs)
    checked = 0
    for k, (got_t, floor) in picks.items():
        got = got_t.double().cpu().numpy()
        want = o[k]
        rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
        bad = ~(np.abs(got - want) <= floor * rms + rtol * np.abs(want))
        if bad.any():
            raise SystemExit(f"parity gate failed on {name} {k}: {int(bad.sum())} elements outside")
        checked += want.size
    return {"checked_elements": int(checked), "rtol": rtol,
            "atol": f"{fe:g} x rms (d_x), {fdt:g} x rms (d_dt), {fs:g} x rms (sums)"}


def conv_fwd_bytes(c) -> int:
    """sx read and out written once, w read once."""
    length = c.n_t + c.d_conv - 1
    io = 2 if c.io == "bf16" else 4
    return c.n_s * c.d_inner * length * io + c.n_s * c.n_t * c.d_inner * io + c.d_inner * c.d_conv * 4


def main_conv_fwd(args):
    import torch
    import ssm_inputs
    import oracle
    from selective_scan_recurrence_amd import ops
    import selective_scan_recurrence_amd as ssm

    ssm.load()
    dev = torch.device("cuda:0")
    c = ssm_inputs.conv_config(args.config)
    step_bytes = conv_fwd_bytes(c)
    copies = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = []
    for _ in range(copies):
        t = {"sx": _dev(c.sx, dev), "w": _dev(c.w, dev)}
        t["out"] = torch.empty(c.n_s, c.n_t, c.d_inner, dtype=t["sx"].dtype, device=dev)
        sets.append(t)

    def step(t):
        return ops.conv_fwd(t["sx"], t["w"], apply_silu=c.apply_silu, out=t["out"])

    got = step(sets[0])
    torch.cuda.synchronize()
    # parity gate: every output element
    want = oracle.conv_fwd(c.sx.value, c.w.value, apply_silu=c.apply_silu)
    g = got.double().cpu().numpy()
    rtol, atol = (2e-2, 1e-3) if c.io == "bf16" else (1e-4, 1e-5)
    bad = ~(np.abs(g - want) <= atol + rtol * np.abs(want))
    if bad.any():
        raise SystemExit(f"parity gate failed on {args.config}: {int(bad.sum())} elements")
    parity = {"checked_elements": int(want.size), "rtol": rtol, "atol": atol}

    for k in range(args.warmup):
        step(sets[k % copies])
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, step, sets, copies, args.steps)
    spread = call_distribution(torch, step, sets, copies)
    avg_s = ms_per_step * 1e-3
    gbs = step_bytes / avg_s / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "ssm_conv_fwd (one launch)", "call_us": round(avg_s * 1e6, 3), "call_spread": spread,
            "floors_us": {"hbm": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)},
            "algorithmic_bytes": step_bytes}
    line = {
        "metric": "ssm_conv forward effective HBM GB/s (% of peak), 1 GPU", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": c.io,
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "n_seqs": c.n_s,
                   "n_tokens": c.n_t, "d_inner": c.d_inner, "d_conv": c.d_conv,
                   "apply_silu": c.apply_silu, "input_copies": copies},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "roofline": roof, "parity": parity,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        reps, sec = 0, 0.0
        ch = 1024
        while reps < 50 and (reps == 0 or sec < 10.0):
            t0 = time.perf_counter()
            oracle.conv_fwd(c.sx.value[:, :ch], c.w.value[:ch], apply_silu=c.apply_silu)
            sec += time.perf_counter() - t0
            reps += 1
        per = sec / reps
        line["cpu_baseline"] = {
            "value": round(step_bytes * ch / c.d_inner / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"first {ch} of {c.d_inner} channels, all sequences and tokens; "
                                        f"{reps} repetitions",
            "seconds": round(sec, 3), "cpu": platform.processor() or platform.machine(),
            "nproc": os.cpu_count()}
    print(json.dumps(line), flush=True)


def conv_bwd_bytes(c) -> int:
    """sx read, dout read, d_sx written (each once), w and d_w."""
    length = c.n_t + c.d_conv - 1
    io = 2 if c.io == "bf16" else 4
    return (c.n_s * c.d_inner * length * (io + 4) + c.n_s * c.n_t * c.d_inner * 4 +
            2 * c.d_inner * c.d_conv * 4)


def cpu_baseline_conv(c, min_seconds=10.0, max_reps=50):
    """The float64 oracle's conv backward on the first 1024 channels, repeated
    until about min_seconds of CPU work."""
    import oracle
    ch = min(1024, c.d_inner)
    sx, w, g = c.sx.value[:, :ch], c.w.value[:ch], c.dout.value[:, :, :ch]
    reps, sec = 0, 0.0
    while reps < max_reps and (reps == 0 or sec < min_seconds):
        t0 = time.perf_counter()
        oracle.conv_bwd(sx, w, g, apply_silu=c.apply_silu)
        sec += time.perf_counter() - t0
        reps += 1
    per = sec / reps
    gbs = conv_bwd_bytes(c) * ch / c.d_inner / per / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {ch} of {c.d_inner} channels, all sequences and tokens; {reps} repetitions",
            "seconds": round(sec, 3), "cpu": platform.processor() or platform.machine(),
            "nproc": os.cpu_count()}


def main_conv_bwd(args):
    import torch
    import ssm_inputs
    import oracle
    from selective_scan_recurrence_amd import ops
    import selective_scan_recurrence_amd as ssm

    ssm.load()
    dev = torch.device("cuda:0")
    c = ssm_inputs.conv_config(args.config)
    step_bytes = conv_bwd_bytes(c)
    copies = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = []
    for _ in range(copies):
        t = {"sx": _dev(c.sx, dev), "w": _dev(c.w, dev), "dout": _dev(c.dout, dev),
             "ws": ops.conv_bwd_workspace(c.n_s, c.n_t, c.d_inner, c.d_conv, dev)}
        length = c.n_t + c.d_conv - 1
        t["dgrad"] = torch.empty(c.n_s * c.d_inner * length + c.d_inner * c.d_conv,
                                 dtype=torch.float32, device=dev)
        sets.append(t)

    def step(t):
        return ops.conv_bwd(t["sx"], t["w"], t["dout"], apply_silu=c.apply_silu, ws=t["ws"],
                            dgrad=t["dgrad"])

    d_sx, d_w = step(sets[0])
    torch.cuda.synchronize()
    # parity gate: every element of sampled channels (each channel's gradients depend on it alone)
    rng = np.random.default_rng(0xB5)
    ch = np.unique(np.concatenate([[0, c.d_inner - 1], rng.choice(c.d_inner, 14, replace=False)]))
    o_sx, o_w = oracle.conv_bwd(c.sx.value[:, ch], c.w.value[ch], c.dout.value[:, :, ch],
                                apply_silu=c.apply_silu)
    hs = torch.as_tensor(ch, device=dev)
    for got_t, want, floor, what in ((d_sx.index_select(1, hs), o_sx, 1e-5, "d_sx"),
                                     (d_w.index_select(0, hs), o_w, 1e-4, "d_w")):
        got = got_t.double().cpu().numpy()
        rms = float(np.sqrt(np.mean(want ** 2)))
        bad = ~(np.abs(got - want) <= floor * rms + 1e-4 * np.abs(want))
        if bad.any():
            raise SystemExit(f"parity gate failed on {args.config} {what}: {int(bad.sum())} elements")
    parity = {"checked_elements": int(o_sx.size + o_w.size), "rtol": 1e-4,
              "atol": "1e-5 x rms (d_sx), 1e-4 x rms (d_w)"}

    for k in range(args.warmup):
        step(sets[k % copies])
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, step, sets, copies, args.steps)
    spread = call_distribution(torch, step, sets, copies)
    avg_s = ms_per_step * 1e-3  # the timed region's mean call duration
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    ach = step_bytes / avg_s / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "ssm_conv_bwd (all launches of one call)", "call_us": round(avg_s * 1e6, 3), "call_spread": spread,
            "floors_us": {"hbm": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)},
            "algorithmic_bytes": step_bytes}
    line = {
        "metric": "ssm_conv backward effective HBM GB/s (% of peak), 1 GPU", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": c.io,
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "n_seqs": c.n_s,
                   "n_tokens": c.n_t, "d_inner": c.d_inner, "d_conv": c.d_conv,
                   "apply_silu": c.apply_silu, "input_copies": copies},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "roofline": roof, "parity": parity,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_conv(c)
    print(json.dumps(line), flush=True)


def decode_bytes(p) -> int:
    """One decode step: the named state rows (and conv-state rows) read and
    written once, x/dt/z read and y written once, B/C and the per-head
    parameters read once."""
    io = 2 if p.io == "bf16" else 4
    S, H, P, N, G, K = p.n_seqs, p.n_head, p.head_dim, p.d_state, p.n_group, p.d_conv
    state = 2 * S * H * P * N * 4
    conv = 2 * S * H * max(K - 1, 0) * 4
    acts = S * H * P * io * (3 if p.value("z") is not None else 2) + S * H * io
    bc = 2 * S * G * N * io
    params = (H * N if p.a_per_state else H) * 4 + (H * 4 if p.has_D else 0) + H * K * 4 + S * 4
    if p.value("dt_bias") is not None:
        params += H * 4
    return state + conv + acts + bc + params


def cpu_baseline_decode(p, min_seconds=10.0, max_reps=200):
    """The float64 oracle's decode step on the whole batch, repeated until
    about min_seconds of CPU work."""
    import oracle
    S, H, P, N, G = p.n_seqs, p.n_head, p.head_dim, p.d_state, p.n_group
    args = (p.value("s"), p.value("x").reshape(S, H, P), p.value("dt").reshape(S, H), p.value("A"),
            p.value("B").reshape(S, G, N), p.value("C").reshape(S, G, N), p.value("D"), p.ids)
    kw = dict(dt_bias=p.value("dt_bias"), z=p.value("z"),
              conv_w=p.value("conv_w") if p.d_conv else None,
              conv_state=p.value("conv_state") if p.d_conv else None, dt_softplus=p.dt_softplus)
    reps, sec = 0, 0.0
    while reps < max_reps and (reps == 0 or sec < min_seconds):
        t0 = time.perf_counter()
        oracle.state_update(*args, **kw)
        sec += time.perf_counter() - t0
        reps += 1
    per = sec / reps
    return {"value": round(decode_bytes(p) / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"the whole batch; {reps} repetitions",
            "seconds": round(sec, 3), "cpu": platform.processor() or platform.machine(),
            "nproc": os.cpu_count()}


def main_decode(args):
    import torch
    import ssm_inputs
    import oracle
    from selective_scan_recurrence_amd import ops
    import selective_scan_recurrence_amd as ssm

    ssm.load()
    dev = torch.device("cuda:0")
    p = ssm_inputs.decode_config(args.config)
    S, H, P, N, G = p.n_seqs, p.n_head, p.head_dim, p.d_state, p.n_group
    desc = ops.make_desc(n_seqs=S, n_tokens=1, n_head=H, head_dim=P, d_state=N, n_group=G,
                         n_state_rows=p.n_state_rows, a_per_state=p.a_per_state, d_conv=p.d_conv,
                         io=p.io, has_D=p.has_D, dt_softplus=p.dt_softplus)
    step_bytes = decode_bytes(p)
    copies = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = []
    for _ in range(copies):
        t = {k: _dev(s_, dev) for k, s_ in p.t.items()}
        t["ids"] = torch.from_numpy(p.ids).to(dev)
        t["y"] = torch.empty(S, H, P, dtype=ops.TORCH_IO[desc.io_dtype], device=dev)
        sets.append(t)

    def step(t):
        return ops.state_update(desc, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                                t["ids"], dt_bias=t.get("dt_bias"), z=t.get("z"),
                                conv_w=t.get("conv_w"), conv_state=t.get("conv_state"), y=t["y"])

    # parity gate on the first call: every element of y and of the state rows
    y = step(sets[0])
    torch.cuda.synchronize()
    cs = p.value("conv_state") if p.d_conv else None
    y_o, s_o, cs_o = oracle.state_update(
        p.value("s"), p.value("x").reshape(S, H, P), p.value("dt").reshape(S, H), p.value("A"),
        p.value("B").reshape(S, G, N), p.value("C").reshape(S, G, N), p.value("D"), p.ids,
        dt_bias=p.value("dt_bias"), z=p.value("z"), conv_w=p.value("conv_w") if p.d_conv else None,
        conv_state=cs, dt_softplus=p.dt_softplus)
    rtol, atol = (2e-2, 1e-3) if p.io == "bf16" else (1e-4, 1e-5)
    checks = [(y.double().cpu().numpy(), y_o, rtol, atol, "y"),
              (sets[0]["s"].double().cpu().numpy(), s_o, 1e-4, 1e-5, "state")]
    if p.d_conv:
        checks.append((sets[0]["conv_state"].double().cpu().numpy(), cs_o, 0.0, 0.0, "conv state"))
    for got, want, rt, at, what in checks:
        bad = ~(np.abs(got - want) <= at + rt * np.abs(want))
        if bad.any():
            raise SystemExit(f"parity gate failed on {args.config} {what}: {int(bad.sum())} elements")
    parity = {"checked_elements": int(sum(c[1].size for c in checks)), "rtol_y": rtol,
              "atol_y": atol, "state": "rtol 1e-4, atol 1e-5", "conv_state": "exact"}

    for k in range(args.warmup):
        step(sets[k % copies])
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, step, sets, copies, args.steps)
    spread = call_distribution(torch, step, sets, copies)
    avg_s = ms_per_step * 1e-3  # the timed region's mean call duration
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    ach = step_bytes / avg_s / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "selective_state_update", "call_us": round(avg_s * 1e6, 3), "call_spread": spread,
            "floors_us": {"hbm": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)},
            "algorithmic_bytes": step_bytes}
    line = {
        "metric": "selective-scan decode step effective HBM GB/s (% of peak) + channel-tokens/s, 1 GPU",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.io,
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "n_seqs": S,
                   "n_head": H, "head_dim": P, "d_state": N, "d_conv": p.d_conv,
                   "input_copies": copies},
        "channel_tokens_per_s": round(S * H * P / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "roofline": roof, "parity": parity,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(p)
    print(json.dumps(line), flush=True)


def timed_steps(torch, step, sets, copies, steps):
    """Times exactly `steps` calls of step(sets[k % copies]), queued back to
    back: two events on the library's stream (torch's current stream)
    bracket the whole region.  Returns (ms per step, wall seconds)."""
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_begin.record()
    for k in range(steps):
        step(sets[k % copies])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return t_begin.elapsed_time(t_end) / steps, wall


def call_distribution(torch, step, sets, copies, n=30):
    """A separate pass after the timed region: n calls, each bracketed by its
    own pair of events, for the spread of single-call durations (median,
    p10, p90, in us).  An event pair adds a few us of its own to each call,
    so these figures sit slightly above the timed region's mean."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for k, (a, b) in enumerate(pairs):
        a.record()
        step(sets[k % copies])
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    return {"median_us": round(float(np.median(us)), 3), "p10_us": round(float(np.percentile(us, 10)), 3),
            "p90_us": round(float(np.percentile(us, 90)), 3), "calls": n,
            "how": "one event pair per call, separate pass after the timed region"}


def varlen_bytes(p) -> int:
    """Each input read once, each output written once, over the packed token axis."""
    io = 2 if p.io == "bf16" else 4
    T, S, H, N, K = p.total_tokens, p.n_seqs, p.n_head, p.d_state, p.d_conv
    x = y = z = T * H * io
    dt = T * H * io
    bc = 2 * T * N * io
    params = (H * N + H + H * K + H) * 4           # A, D, conv_w, dt_bias
    states = 2 * S * H * N * 4 + 2 * S * H * (K - 1) * 4   # state and conv state, in and out
    return x + y + z + dt + bc + params + states + S * 4 + (S + 1) * 4


def valu_ops_ext(p):
    """valu_ops_per_channel_token plus the extras per channel-token: the bias
    (add), softplus (exp, log: 3 ops and 2 transcendentals) and the gate
    SiLU(z) * y (mul, add, mul and exp, rcp)."""
    ops, trans = valu_ops_per_channel_token(p)
    return ops + 1 + 3 + 3, trans + 2 + 2


def valu_slots_ext(p) -> float:
    ops, trans = valu_ops_ext(p)
    return ops + TRANS_COST * trans


def _oracle_ext_heads(p, heads):
    import oracle
    v = lambda n: None if p.value(n) is None else p.value(n).astype(np.float64)
    pk = lambda n: v(n)[0][:, heads]
    return oracle.scan_fwd_ext(v("s")[:, heads], pk("x"), pk("dt"), v("A")[heads], v("B")[0], v("C")[0],
                               v("D")[heads], p.ids, cu_seqlens=p.cu_seqlens,
                               dt_bias=v("dt_bias")[heads], z=pk("z"), conv_w=v("conv_w")[heads],
                               conv_state=v("conv_state")[:, heads], dt_softplus=p.dt_softplus,
                               n_threads=oracle.default_threads())


def main_varlen(args):
    """C9: the fused forward over packed sequences of mixed lengths with the
    dt bias and the z gate (selective_scan_fwd_ext)."""
    import torch
    import oracle
    import ssm_inputs
    from selective_scan_recurrence_amd import ops
    import selective_scan_recurrence_amd as ssm

    ssm.load()
    dev = torch.device("cuda:0")
    name = args.config
    p = ssm_inputs.varlen_config(name)
    desc = ops.make_desc(n_seqs=p.n_seqs, n_tokens=p.n_tokens, n_head=p.n_head, d_state=p.d_state,
                         n_state_rows=p.n_state_rows, d_conv=p.d_conv,
                         chunk=0 if args.chunk is None else args.chunk, io=p.io, has_D=p.has_D,
                         dt_softplus=p.dt_softplus)
    step_bytes = varlen_bytes(p)
    copies = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = []
    for _ in range(copies):
        t = {k: _dev(s, dev) for k, s in p.t.items()}
        t["ids"] = torch.from_numpy(p.ids).to(dev)
        t["cu"] = torch.from_numpy(p.cu_seqlens).to(dev)
        t["ws"] = ops.workspace(desc, False, dev)
        t["out"] = torch.empty(ssm.ssm_scan_ext_out_bytes(desc, ssm.make_ext(cu_seqlens=1, total_tokens=p.total_tokens))[0],
                               dtype=torch.uint8, device=dev)
        t["cso"] = torch.empty(p.n_seqs, p.n_head, p.d_conv - 1, dtype=torch.float32, device=dev)
        sets.append(t)

    def step(t):
        return ops.scan_fwd_ext(desc, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["ids"],
                                dt_bias=t["dt_bias"], z=t["z"], cu_seqlens=t["cu"],
                                total_tokens=p.total_tokens, conv_w=t["conv_w"],
                                conv_state=t["conv_state"], want_conv_state=True, ws=t["ws"], out=t["out"])

    res = step(sets[0])
    torch.cuda.synchronize()
    # parity gate: every token of sampled channels against the oracle
    rng = np.random.default_rng(0xB9)
    heads = np.unique(np.concatenate([[0, p.n_head - 1], rng.choice(p.n_head, 8, replace=False)]))
    y_o, st_o, cs_o = _oracle_ext_heads(p, heads)
    hs = torch.as_tensor(heads, device=dev)
    rtol, atol = 2e-2, 1e-3
    # y's absolute floor scales with |SiLU(z)|: the gate multiplies an fp32 y
    # that carries the ungated error
    zg = p.value("z")[0][:, heads].astype(np.float64)
    gate = np.maximum(1.0, np.abs(zg / (1.0 + np.exp(-zg))))
    checked = 0
    for got, want, what, sc in ((res.y.index_select(1, hs), y_o, "y", gate),
                                (res.state.index_select(1, hs), st_o, "state", 1.0),
                                (res.conv_state.index_select(1, hs), cs_o, "conv_state", 1.0)):
        g = got.double().cpu().numpy()
        bad = ~(np.abs(g - want) <= atol * sc + rtol * np.abs(want))
        if bad.any():
            raise SystemExit(f"parity gate failed on {name} {what}: {int(bad.sum())} elements outside "
                             f"rtol={rtol} atol={atol}")
        checked += want.size
    if ssm.ssm_get_device_error(sets[0]["ws"]):
        raise SystemExit(f"{name}: device error word set")
    parity = {"checked_elements": int(checked), "rtol": rtol, "atol": atol,
              "atol_y": "1e-3 x max(1, |SiLU(z)|)"}

    for k in range(args.warmup):
        step(sets[k % copies])
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, step, sets, copies, args.steps)
    spread = call_distribution(torch, step, sets, copies)
    avg_s = ms_per_step * 1e-3  # the timed region's mean call duration
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    ch_tok = p.total_tokens * p.n_head
    slots = valu_slots_ext(p) * ch_tok
    floors = {"hbm": step_bytes / (HBM_PEAK_GBS * 1e9), "alu": slots / (VALU_PEAK_T * 1e12)}
    if floors["alu"] >= floors["hbm"]:
        ach = slots / avg_s / 1e12
        roof = {"bound": "alu", "achieved": round(ach, 3), "peak": VALU_PEAK_T, "unit": "T VALU-slots/s",
                "frac": round(ach / VALU_PEAK_T, 4)}
    else:
        ach = step_bytes / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": measured_traffic(name),
                 "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                 "kernel": "selective_scan_fwd_ext (all launches of one call)",
                 "call_us": round(avg_s * 1e6, 3), "call_spread": spread,
                 "floors_us": {k: round(v * 1e6, 2) for k, v in floors.items()},
                 "algorithmic_bytes": step_bytes, "valu_slots": int(slots),
                 "issue_model": issue_model(valu_ops_ext(p), ch_tok, avg_s)})
    lengths = np.diff(p.cu_seqlens).tolist()
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "n_seqs": p.n_seqs,
                   "total_tokens": p.total_tokens, "lengths": lengths, "n_head": p.n_head,
                   "d_state": p.d_state, "d_conv": p.d_conv, "chunk": desc.chunk,
                   "input_copies": copies},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "channel_tokens_per_s": round(ch_tok / (ms_per_step * 1e-3), 1),
        "roofline": roof, "parity": parity, "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        n = 1024
        sub = np.arange(n)
        reps, sec = 0, 0.0
        while reps < 50 and (reps == 0 or sec < 10.0):
            t1 = time.perf_counter()
            _oracle_ext_heads(p, sub)
            sec += time.perf_counter() - t1
            reps += 1
        per = sec / reps
        line["cpu_baseline"] = {
            "value": round(step_bytes * n / p.n_head / per / 1e9, 4), "unit": "GB/s",
            "cores": oracle.threads_used(n, oracle.default_threads()), "kind": "oracle",
            "sample": f"first {n} of {p.n_head} channels, all sequences and tokens; {reps} repetitions",
            "seconds": round(sec, 3), "channel_tokens_per_s": round(p.total_tokens * n / per, 1),
            "cpu": platform.processor() or platform.machine(), "nproc": os.cpu_count()}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C2", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk", type=int, default=None, help="override the time chunk (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 1 GiB device copies (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: there is no multi-GPU path (asked for "
              f"--gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.config == "C5":
        main_conv_bwd(args)
        return
    if args.config == "C11":
        main_conv_fwd(args)
        return
    if args.config in ("C6", "C7"):
        main_decode(args)
        return
    if args.config == "C9":
        main_varlen(args)
        return
    import torch
    import ssm_inputs
    from selective_scan_recurrence_amd import ops
    import selective_scan_recurrence_amd as ssm

    ssm.load()
    dev = torch.device("cuda:0")
    name = args.config
    backward = name in ("C4", "C8", "C10")
    p = ssm_inputs.config(name)
    desc = ops.make_desc(n_seqs=p.n_seqs, n_tokens=p.n_tokens, n_head=p.n_head,
                         head_dim=p.head_dim, d_state=p.d_state, n_group=p.n_group,
                         n_state_rows=p.n_state_rows, a_per_state=p.a_per_state,
                         d_conv=p.d_conv, chunk=p.chunk if args.chunk is None else args.chunk,
                         io=p.io, has_D=p.has_D, dt_softplus=p.dt_softplus)
    step_bytes = algorithmic_bytes(p, backward)
    copies = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = []
    for _ in range(copies):
        t = {k: _dev(s, dev) for k, s in p.t.items()}
        t["ids"] = torch.from_numpy(p.ids).to(dev)
        t["ws"] = ops.workspace(desc, backward, dev)
        if backward:
            t["dout"] = torch.cat([t.pop("dy").reshape(-1).view(torch.uint8),
                                   t.pop("dstate").reshape(-1).view(torch.uint8)])
            t["out"] = torch.empty(ssm.ssm_scan_dgrad_layout(desc)[0], dtype=torch.uint8, device=dev)
        else:
            t["out"] = torch.empty(ssm.ssm_scan_out_bytes(desc), dtype=torch.uint8, device=dev)
        sets.append(t)

    def step(t):
        if backward:
            return ops.scan_bwd(desc, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                                t["ids"], t["dout"], ws=t["ws"], dgrad=t["out"],
                                conv_w=t.get("conv_w"), conv_state=t.get("conv_state"))
        return ops.scan_fwd(desc, t["s"], t["x"], t["dt"], t["A"], t["B"], t["C"], t.get("D"),
                            t["ids"], conv_w=t.get("conv_w"), conv_state=t.get("conv_state"),
                            ws=t["ws"], out=t["out"])

    res = step(sets[0])
    torch.cuda.synchronize()
    parity = parity_gate_bwd(name, p, res[1]) if backward else parity_gate(name, p, res)

    for k in range(args.warmup):
        step(sets[k % copies])
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, step, sets, copies, args.steps)
    spread = call_distribution(torch, step, sets, copies)
    avg_s = ms_per_step * 1e-3  # the timed region's mean call duration
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    ch_tok = p.n_seqs * p.n_tokens * p.n_head * p.head_dim
    floors = {"hbm": step_bytes / (HBM_PEAK_GBS * 1e9)}
    if uses_ssd(p):
        flops = ssd_bwd_mfma_flops(p) if backward else ssd_mfma_flops(p)
        floors["mfma"] = flops / (MFMA_BF16_PEAK_T * 1e12)
    else:
        slots = valu_slots_per_channel_token(p, backward) * ch_tok
        floors["alu"] = slots / (VALU_PEAK_T * 1e12)
    bound = max(floors, key=floors.get)
    if bound == "hbm":
        ach = step_bytes / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    elif bound == "mfma":
        ach = flops / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_T,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_T, 4)}
    else:
        ach = slots / avg_s / 1e12
        roof = {"bound": "alu", "achieved": round(ach, 3), "peak": VALU_PEAK_T,
                "unit": "T VALU-slots/s", "frac": round(ach / VALU_PEAK_T, 4)}
    roof.update({"traffic": measured_traffic(name), "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                 "kernel": f"{'selective_scan_bwd' if backward else 'selective_scan_fwd'} "
                           "(all launches of one call)",
                 "call_us": round(avg_s * 1e6, 3), "call_spread": spread,
                 "floors_us": {k: round(v * 1e6, 2) for k, v in floors.items()},
                 "algorithmic_bytes": step_bytes})
    if "alu" in floors:
        roof["valu_slots"] = int(slots)
        roof["issue_model"] = issue_model(valu_ops_per_channel_token(p, backward), ch_tok, avg_s)
    if "mfma" in floors:
        roof["mfma_flops"] = int(flops)
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if p.io == "f32" else "bf16",
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": f"{name}: {WORKLOADS[name]}", "n_seqs": p.n_seqs,
                   "n_tokens": p.n_tokens, "n_head": p.n_head, "head_dim": p.head_dim,
                   "d_state": p.d_state, "n_group": p.n_group, "d_conv": p.d_conv,
                   "chunk": SSD_Q if uses_ssd(p) else desc.chunk, "input_copies": copies},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "channel_tokens_per_s": round(ch_tok / (ms_per_step * 1e-3), 1),
        "roofline": roof,
        "parity": parity,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(name, p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
