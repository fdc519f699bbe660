"""Pins for the oracle's forward extras (``oracle.scan_fwd_ext``): the dt bias
and SiLU(z) gate of the per-token step of "mambazip mamba1/model.rs"
(forward_impl), and sequences packed on one token axis (the RWKV-6/7 shapes of "ggmlR
tests/testthat/test-ssm-rwkv.R", generalised to per-sequence lengths).  Each is checked against the
separately pinned equal-length scan, invariants of the recurrence, or exact
special cases -- never against its own formula retyped.  Each test names the
mistake it would catch.  CPU only.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import ssm_inputs


def V(p, name):
    a = p.value(name)
    return None if a is None else a.astype(np.float64)


def _varlen(form, lengths, seed, **kw):
    if form == "m1":
        base = dict(n_head=6, d_state=5, d_conv=4, conv_state_std=0.7, A_kind="uniform", A_range=(0.2, 2.0))
    else:
        base = dict(n_head=4, head_dim=3, d_state=4, n_group=2, a_per_state=False, d_conv=0,
                    A_kind="uniform", A_range=(0.2, 2.0))
    base.update(kw)
    return ssm_inputs.make_varlen_problem(lengths=lengths, io="f32", seed=seed, h0_std=0.5,
                                          n_state_rows=len(lengths) + 2, **base)


def _ext(p, cu=True, **kw):
    v = lambda n: V(p, n)
    x, dt, B, C = v("x")[0], v("dt")[0], v("B")[0], v("C")[0]
    return oracle.scan_fwd_ext(v("s"), x, dt, v("A"), B, C, v("D"), p.ids,
                               cu_seqlens=p.cu_seqlens if cu else None,
                               conv_w=v("conv_w") if p.d_conv else None,
                               conv_state=v("conv_state") if p.d_conv else None, **kw)


# --------------------------------------------------------------------------
# Equal spans reproduce the batched scan: sequences of L tokens packed at
# i*L equal scan_fwd on the [S][L] layout, element for element.  Catches: a
# wrong offset into the packed axis, a sequence read from another's tokens or
# state row, a conv window that starts at the wrong token.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["m1", "m2"])
def test_ext_equal_spans_equal_batched(form):
    S, L = 4, 9
    p = _varlen(form, [L] * S, 61)
    y, st, cso = _ext(p, dt_softplus=True)
    sh = lambda a: a.reshape((S, L) + a.shape[1:])
    yb, stb, csb = oracle.scan_fwd(V(p, "s"), sh(V(p, "x")[0]), sh(V(p, "dt")[0]), V(p, "A"),
                                   sh(V(p, "B")[0]), sh(V(p, "C")[0]), V(p, "D"), p.ids,
                                   conv_w=V(p, "conv_w") if p.d_conv else None,
                                   conv_state=V(p, "conv_state") if p.d_conv else None,
                                   dt_softplus=True)
    np.testing.assert_allclose(sh(y), yb, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(st, stb, rtol=1e-15, atol=1e-15)
    if p.d_conv:
        assert np.array_equal(cso, csb)


# --------------------------------------------------------------------------
# Splitting every sequence in two and running the pieces as two packed calls
# -- the second from the first's final states and conv states -- gives the
# unsplit scan.  The first pieces have lengths 0, 1, 2 (shorter than the
# conv window) and longer.  Catches: a conv ring that drops or reorders
# entries of a short sequence, a final state not taken after the last token,
# a span that runs one token long or short.
# --------------------------------------------------------------------------
def test_ext_split_chain_equals_unsplit():
    S, L = 5, 11
    first = np.array([0, 1, 2, 6, 11])
    p = _varlen("m1", [L] * S, 67)
    x, dt, B, C = (V(p, n)[0].reshape((S, L) + V(p, n)[0].shape[1:]) for n in ("x", "dt", "B", "C"))
    kw = dict(conv_w=V(p, "conv_w"), dt_softplus=True)
    y_full, st_full, cs_full = oracle.scan_fwd(V(p, "s"), x, dt, V(p, "A"), B, C, V(p, "D"), p.ids,
                                               conv_state=V(p, "conv_state"), **kw)

    def pack(a, sl):
        return np.concatenate([a[i, sl[i]] for i in range(S)], axis=0)
    sl1 = [slice(0, f) for f in first]
    sl2 = [slice(f, L) for f in first]
    cu1 = np.concatenate([[0], np.cumsum(first)])
    cu2 = np.concatenate([[0], np.cumsum(L - first)])
    y1, st1, cs1 = oracle.scan_fwd_ext(V(p, "s"), pack(x, sl1), pack(dt, sl1), V(p, "A"), pack(B, sl1),
                                       pack(C, sl1), V(p, "D"), p.ids, cu_seqlens=cu1,
                                       conv_state=V(p, "conv_state"), **kw)
    ident = np.arange(S, dtype=np.int32)
    y2, st2, cs2 = oracle.scan_fwd_ext(st1, pack(x, sl2), pack(dt, sl2), V(p, "A"), pack(B, sl2),
                                       pack(C, sl2), V(p, "D"), ident, cu_seqlens=cu2,
                                       conv_state=cs1, **kw)
    for i in range(S):
        got = np.concatenate([y1[cu1[i]:cu1[i + 1]], y2[cu2[i]:cu2[i + 1]]])
        np.testing.assert_allclose(got, y_full[i], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st2, st_full, rtol=1e-12, atol=1e-13)
    assert np.array_equal(cs2, cs_full)


# --------------------------------------------------------------------------
# A zero-length sequence returns its state row and conv-state row unchanged
# and leaves the others' results as if it were absent.  Catches: an empty
# span that still reads a token, a conv state taken from the wrong row.
# --------------------------------------------------------------------------
def test_ext_zero_length_sequences():
    lengths = [5, 0, 7, 0, 3]
    p = _varlen("m1", lengths, 71)
    y, st, cso = _ext(p)
    for i, n in enumerate(lengths):
        if n == 0:
            assert np.array_equal(st[i], V(p, "s")[p.ids[i]])
            assert np.array_equal(cso[i], V(p, "conv_state")[p.ids[i]])
    keep = [i for i, n in enumerate(lengths) if n]
    q = _varlen("m1", lengths, 71)
    q.ids = p.ids[keep]
    q.cu_seqlens = np.concatenate([[0], np.cumsum(np.asarray(lengths)[keep])]).astype(np.int32)
    y2, st2, cs2 = _ext(q)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(st2, st[keep])
    np.testing.assert_array_equal(cs2, cso[keep])


# --------------------------------------------------------------------------
# The gate multiplies y by SiLU(z) = z * logistic(z) (scipy's expit) and
# leaves the states alone; the bias is added to dt before softplus: (dt,
# bias) equals (dt + bias, none), and with softplus on it equals softplus(dt
# + bias) (numpy's logaddexp, all arguments below 20) given with softplus
# off.  Catches: a gate of logistic(z) alone, a gate applied before D.u is
# added or to the state, the bias added after softplus or per channel.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["m1", "m2"])
def test_ext_gate_and_bias(form):
    p = _varlen(form, [4, 9, 1, 6], 73, )
    rng = np.random.default_rng(7)
    T, H, P = V(p, "x")[0].shape
    z = rng.normal(size=(T, H, P))
    bias = rng.uniform(-1, 1, H)
    y0, s0, c0 = _ext(p)
    yg, sg, cg = _ext(p, z=z)
    np.testing.assert_allclose(yg, y0 * z * expit(z), rtol=1e-13, atol=1e-15)
    assert np.array_equal(sg, s0)

    v = lambda n: V(p, n)
    base = (v("s"), v("x")[0])
    rest = (v("A"), v("B")[0], v("C")[0], v("D"), p.ids)
    kw = dict(cu_seqlens=p.cu_seqlens, conv_w=v("conv_w") if p.d_conv else None,
              conv_state=v("conv_state") if p.d_conv else None)
    dt = v("dt")[0]
    y_b, s_b, _ = oracle.scan_fwd_ext(*base, dt, *rest, dt_bias=bias, **kw)
    y_s, s_s, _ = oracle.scan_fwd_ext(*base, dt + bias[None, :], *rest, **kw)
    np.testing.assert_allclose(y_b, y_s, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s_b, s_s, rtol=1e-14, atol=1e-15)
    y_sp, s_sp, _ = oracle.scan_fwd_ext(*base, dt, *rest, dt_bias=bias, dt_softplus=True, **kw)
    y_pre, s_pre, _ = oracle.scan_fwd_ext(*base, np.logaddexp(0.0, dt + bias[None, :]), *rest, **kw)
    np.testing.assert_allclose(y_sp, y_pre, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s_sp, s_pre, rtol=1e-12, atol=1e-14)
