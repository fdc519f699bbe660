"""Pins for the float64 oracle: checks against what the pages and the
mathematics fix, never against the oracle's own formula retyped.

Each test names the mistake it would catch.  CPU only.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import ssm_inputs


def V(p, name):
    """A stored input as float64 (exact), or None."""
    a = p.value(name)
    return None if a is None else a.astype(np.float64)


def _tiny(seed, **kw):
    base = dict(n_seqs=2, n_tokens=9, n_head=3, d_state=4, d_conv=0, io="f32",
                seed=seed, h0_std=0.5, A_kind="uniform", A_range=(0.2, 2.0))
    base.update(kw)
    return ssm_inputs.make_problem(**base)


def _fwd(p, **over):
    v = {k: V(p, k) for k in ("s", "x", "dt", "A", "B", "C", "D", "conv_w", "conv_state")}
    v.update(over)
    return oracle.scan_fwd(v["s"], v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], p.ids,
                           conv_w=v["conv_w"], conv_state=v["conv_state"],
                           dt_softplus=p.dt_softplus)


# --------------------------------------------------------------------------
# Depthwise conv ("ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv test
# against a convolution computed in R): each output channel is the valid
# cross-correlation of that channel's input row (the d_conv-1 earlier inputs
# followed by the tokens) with that channel's taps, so the last tap meets
# the newest input.  numpy's correlate computes it channel by channel.
# Catches: reversed tap order, an off-by-one in the window, a transposed layout.
# --------------------------------------------------------------------------
def _depthwise_reference(sx, w):
    """sx [n_s][d_inner][d_conv-1+n_t], w [d_inner][d_conv] -> [n_s][n_t][d_inner]."""
    n_s, d_inner, _ = sx.shape
    out = np.stack([np.stack([np.correlate(sx[s, ch], w[ch], mode="valid") for ch in range(d_inner)],
                             axis=-1) for s in range(n_s)])
    return out


@pytest.mark.parametrize("d_conv,d_inner,n_t,n_s", [(3, 5, 6, 2), (4, 3, 9, 1), (1, 2, 3, 1),
                                                    (2, 4, 1, 3)])
def test_conv_matches_depthwise_correlation(d_conv, d_inner, n_t, n_s):
    rng = np.random.default_rng(0x2C0)
    sx = rng.uniform(-1, 1, (n_s, d_inner, d_conv - 1 + n_t))
    w = rng.uniform(-1, 1, (d_inner, d_conv))
    got = oracle.conv_fwd(sx, w)
    assert got.shape == (n_s, n_t, d_inner)
    np.testing.assert_allclose(got, _depthwise_reference(sx, w), rtol=1e-14, atol=1e-15)
    # a single unit tap at position j picks the input j places after the window start
    for j in range(d_conv):
        e = np.zeros((d_inner, d_conv))
        e[:, j] = 1.0
        np.testing.assert_array_equal(oracle.conv_fwd(sx, e),
                                      np.transpose(sx[:, :, j:j + n_t], (0, 2, 1)))
    got_silu = oracle.conv_fwd(sx, w, apply_silu=True)
    np.testing.assert_allclose(got_silu, got * expit(got), rtol=1e-13, atol=1e-15)


def test_fused_conv_silu_feeds_scan():
    """With B = C = 0 the scan adds nothing and D = 1 passes u through, so
    y = SiLU(conv([conv_state | x])) by the page's brute force.
    Catches: tap order, ignoring the conv state, SiLU applied to the wrong value."""
    p = ssm_inputs.make_problem(n_seqs=2, n_tokens=7, n_head=3, d_state=2, d_conv=4,
                                io="f32", seed=3, h0_std=1.0, conv_state_std=1.0,
                                n_state_rows=3, ids=np.array([2, 0], np.int32))
    zeros = np.zeros_like(V(p, "B"))
    y, st, cso = _fwd(p, B=zeros, C=zeros, D=np.ones(3))
    x, cs, w = (V(p, k).astype(np.float64) for k in ("x", "conv_state", "conv_w"))
    x = x[..., 0]
    for i, r in enumerate(p.ids):
        sx = np.concatenate([cs[r], x[i].T], axis=1)[None]    # [1][H][K-1+L]
        pre = _depthwise_reference(sx, w)[0]
        np.testing.assert_allclose(y[i, :, :, 0], pre * expit(pre), rtol=1e-13, atol=1e-15)
        # conv_state_out: the last K-1 inputs, oldest first
        np.testing.assert_array_equal(cso[i], sx[0][:, -3:])


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["m1", "m2"])
def test_A_zero_is_cumulative_sum(form):
    """A = 0 => decay 1 => h_t = h0 + sum_{tau<=t} dt B u; y = C.h_t + D u.
    Catches: dt or u dropped from the input term, B and C swapped, y read from
    h_{t-1}, a dropped D term, a wrong head-to-group map."""
    if form == "m1":
        p = _tiny(21)
        A0 = np.zeros_like(V(p, "A"))
    else:
        p = _tiny(22, head_dim=2, n_head=4, n_group=2, a_per_state=False)
        A0 = np.zeros_like(V(p, "A"))
    y, st, _ = _fwd(p, A=A0)
    x, dt, B, C, D, s = (V(p, k) for k in ("x", "dt", "B", "C", "D", "s"))
    S, L, H, P = x.shape
    G = B.shape[2]
    for h in range(H):
        g = h // (H // G)
        for i in range(S):
            h0 = s[p.ids[i], h]                                         # [P][N]
            inc = dt[i, :, h, None, None] * x[i, :, h, :, None] * B[i, :, g, None, :]  # [L][P][N]
            hist = h0[None] + np.cumsum(inc, axis=0)
            y_ref = np.einsum("tpn,tn->tp", hist, C[i, :, g]) + D[h] * x[i, :, h]
            np.testing.assert_allclose(y[i, :, h], y_ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(st[i, h], hist[-1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("form", ["m1", "m2"])
def test_zero_input_is_pure_decay(form):
    """x = 0 => h_t = exp(A * sum_{tau<=t} dt) h0 and y = C.h_t.
    Catches: a sign error in the exponent, decay applied after instead of
    before the step, the per-state vs per-head A layout."""
    p = _tiny(31) if form == "m1" else _tiny(32, head_dim=3, a_per_state=False)
    y, st, _ = _fwd(p, x=np.zeros_like(V(p, "x")))
    dt, A, C, s = (V(p, k) for k in ("dt", "A", "C", "s"))
    S, L, H = dt.shape
    for i in range(S):
        for h in range(H):
            An = A[h] if A.ndim == 2 else np.full(s.shape[3], A[h])
            cum = np.cumsum(dt[i, :, h])                               # [L]
            hist = np.exp(cum[:, None, None] * An[None, None, :]) * s[p.ids[i], h][None]
            np.testing.assert_allclose(y[i, :, h], np.einsum("tpn,tn->tp", hist, C[i, :, 0]),
                                       rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(st[i, h], hist[-1], rtol=1e-12, atol=1e-14)


def test_dt_zero_pins_state_ids_exactly():
    """dt = 0 => decay 1 and no input: the final state of sequence i is row
    ids[i] of s bit for bit, written to row i; y = C.h0 + D u.
    Catches: scattering instead of gathering, writing the state to row ids[i],
    any offset error in the state block.  Repeated ids are allowed."""
    p = ssm_inputs.make_problem(n_seqs=4, n_tokens=5, n_head=3, d_state=4, d_conv=0, io="f32",
                                seed=41, n_state_rows=6, ids=np.array([5, 2, 2, 0], np.int32))
    s = (np.arange(6 * 3 * 4, dtype=np.float64).reshape(6, 3, 1, 4) + 1.0) * 0.25
    y, st, _ = _fwd(p, s=s, dt=np.zeros_like(V(p, "dt")))
    np.testing.assert_array_equal(st, s[p.ids])
    C, D, x = V(p, "C"), V(p, "D"), V(p, "x")
    for i in range(4):
        y_ref = np.einsum("hn,tn->th", s[p.ids[i], :, 0], C[i, :, 0]) + D[None, :] * x[i, :, :, 0]
        np.testing.assert_allclose(y[i, :, :, 0], y_ref, rtol=1e-14, atol=1e-14)


def test_ids_out_of_range_rejected():
    p = _tiny(42)
    with pytest.raises(ValueError):
        oracle.scan_fwd(V(p, "s"), V(p, "x"), V(p, "dt"), V(p, "A"), V(p, "B"),
                        V(p, "C"), V(p, "D"), np.array([0, 2], np.int32))


# --------------------------------------------------------------------------
# Associativity: the same recurrence evaluated three other ways
# --------------------------------------------------------------------------
def _decays_inputs(p):
    """a_t = exp(dt A), b_t = dt B u for the no-conv problem: [S][L][H][P][N]."""
    x, dt, A, B = (V(p, k) for k in ("x", "dt", "A", "B"))
    S, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = np.arange(H) // (H // G)
    An = A if A.ndim == 2 else np.repeat(A[:, None], N, axis=1)
    a = np.exp(dt[:, :, :, None, None] * An[None, None, :, None, :]) * np.ones((1, 1, 1, P, 1))
    b = dt[:, :, :, None, None] * x[..., None] * B[:, :, grp, None, :]
    return a, b


def _hillis_steele(a, b):
    """Inclusive prefix over axis 1 with (a1,b1) o (a2,b2) = (a1 a2, a2 b1 + b2)."""
    a, b = a.copy(), b.copy()
    L = a.shape[1]
    step = 1
    while step < L:
        a_prev = np.ones_like(a)
        b_prev = np.zeros_like(b)
        a_prev[:, step:] = a[:, :-step]
        b_prev[:, step:] = b[:, :-step]
        b = a * b_prev + b
        a = a * a_prev
        step *= 2
    return a, b


@pytest.mark.parametrize("form", ["m1", "m2"])
def test_sequential_equals_associative_prefix(form):
    """Catches any loop-order or indexing error in the oracle's recurrence."""
    p = _tiny(51, n_tokens=37) if form == "m1" else \
        _tiny(52, n_tokens=37, head_dim=2, n_head=4, n_group=2, a_per_state=False)
    y, st, _ = oracle.problem_fwd(p)
    a, b = _decays_inputs(p)
    Ap, Bp = _hillis_steele(a, b)
    h0 = V(p, "s")[p.ids]                                     # [S][H][P][N]
    hist = Ap * h0[:, None] + Bp                                 # [S][L][H][P][N]
    G = V(p, "C").shape[2]
    grp = np.arange(p.n_head) // (p.n_head // G)
    Cg = V(p, "C")[:, :, grp]                                 # [S][L][H][N]
    y_ref = np.einsum("slhpn,slhn->slhp", hist, Cg) + V(p, "D")[None, None, :, None] * V(p, "x")
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st, hist[:, -1], rtol=1e-11, atol=1e-12)


def test_final_state_closed_form():
    """h_T = (prod_t a_t) h0 + sum_tau (prod_{t>tau} a_t) b_tau, written as
    explicit products on a tiny length.  Catches an off-by-one in which
    decays multiply which inputs."""
    p = _tiny(61, n_tokens=6)
    _, st, _ = oracle.problem_fwd(p)
    a, b = _decays_inputs(p)
    L = a.shape[1]
    h0 = V(p, "s")[p.ids]
    ref = np.prod(a, axis=1) * h0
    for tau in range(L):
        ref = ref + np.prod(a[:, tau + 1:], axis=1) * b[:, tau]
    np.testing.assert_allclose(st, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 4, 5, 16, 64])
def test_chunked_with_carries_equals_unchunked(chunk):
    """Each chunk scanned from zero, then the carry (prod a) h_in added:
    the chunked form any parallel kernel uses must equal the sequential one,
    for chunk sizes that do and do not divide the length."""
    p = _tiny(71, n_tokens=23)
    y, st, _ = oracle.problem_fwd(p)
    a, b = _decays_inputs(p)
    L = a.shape[1]
    h_in = V(p, "s")[p.ids]
    hist = np.zeros_like(b)
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        loc = np.zeros_like(h_in)
        decay = np.ones_like(h_in)
        for t in range(c0, c1):
            loc = a[:, t] * loc + b[:, t]
            decay = decay * a[:, t]
            hist[:, t] = loc + decay * h_in
        h_in = hist[:, c1 - 1]
    np.testing.assert_allclose(st, h_in, rtol=1e-12, atol=1e-13)
    y_ref = np.einsum("slhpn,sln->slhp", hist, V(p, "C")[:, :, 0]) + \
        V(p, "D")[None, None, :, None] * V(p, "x")
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-13)


def test_mamba2_scalar_A_equals_mamba1_constant_rows():
    """Cross-form identity: scalar A per head equals a per-state A whose row
    is constant.  Catches the per-head decay read from the wrong head."""
    p = _tiny(81, a_per_state=False)
    y2, st2, _ = oracle.problem_fwd(p)
    A_rows = np.repeat(V(p, "A")[:, None], p.d_state, axis=1)
    y1, st1, _ = _fwd(p, A=A_rows)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(st1, st2)


def test_groups_decompose_into_separate_calls():
    """n_group > 1: heads [g*r, (g+1)*r) read group g of B/C, so each group's
    heads run alone with n_group = 1 give the same result."""
    p = _tiny(91, n_head=6, n_group=3, head_dim=2, a_per_state=False)
    y, st, _ = oracle.problem_fwd(p)
    v = {k: V(p, k) for k in ("s", "x", "dt", "A", "B", "C", "D")}
    for g in range(3):
        hs = slice(2 * g, 2 * g + 2)
        yg, sg, _ = oracle.scan_fwd(v["s"][:, hs], v["x"][:, :, hs], v["dt"][:, :, hs], v["A"][hs],
                                    v["B"][:, :, g:g + 1], v["C"][:, :, g:g + 1], v["D"][hs], p.ids)
        np.testing.assert_array_equal(yg, y[:, :, hs])
        np.testing.assert_array_equal(sg, st[:, hs])


def test_linearity_in_input_and_state():
    """For fixed dt, A, B, C, D the output is linear in (x, h0) jointly."""
    p = _tiny(101)
    q = _tiny(102)
    y1, s1, _ = _fwd(p)
    y2, s2, _ = _fwd(p, x=V(q, "x"), s=V(q, "s") + 0.3)
    y3, s3, _ = _fwd(p, x=V(p, "x") * 2.0 - 3.0 * V(q, "x"),
                     s=V(p, "s") * 2.0 - 3.0 * (V(q, "s") + 0.3))
    np.testing.assert_allclose(y3, 2.0 * y1 - 3.0 * y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, 2.0 * s1 - 3.0 * s2, rtol=1e-12, atol=1e-12)


def test_softplus_flag_equals_pretransformed_dt():
    """dt_softplus uses softplus with the threshold-20 branch; passing the
    transformed dt without the flag must agree."""
    p = _tiny(111)
    raw = V(p, "dt") * 30.0 - 5.0          # spans both branches of the threshold
    p.dt_softplus = True
    y_flag, s_flag, _ = _fwd(p, dt=raw)
    p.dt_softplus = False
    sp = np.where(raw > 20.0, raw, np.log1p(np.exp(np.minimum(raw, 20.0))))
    y_pre, s_pre, _ = _fwd(p, dt=sp)
    np.testing.assert_allclose(y_flag, y_pre, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(s_flag, s_pre, rtol=1e-14, atol=1e-14)


def test_zero_operands_give_zero_output():
    """ggmlR 'the ssm_scan views read back the halves they point at': all-zero
    operands give an all-zero output block."""
    p = _tiny(121)
    z = {k: np.zeros_like(V(p, k)) for k in ("s", "x", "dt", "A", "B", "C", "D")}
    y, st, _ = oracle.scan_fwd(z["s"], z["x"], z["dt"], z["A"], z["B"], z["C"], z["D"], p.ids)
    assert not y.any() and not st.any()
