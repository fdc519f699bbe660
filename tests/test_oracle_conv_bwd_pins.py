"""Pins of the oracle's conv backward (the ggmlR ssm_conv backward).

The page ("ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv backward
block) checks the backward three ways, each restated here against the
float64 oracle:
  * the packed result holds the sx gradient then the weight gradient, so its
    size is nelem(sx) + nelem(w);
  * both gradients equal a central difference of <ssm_conv(sx, w), g>;
  * with loss = sum(output), the weight gradient is the sum of the sx values
    each tap reads.
Added here: the adjoint identities of the linear conv (exact up to
rounding), the SiLU factor at z = 0 (a half), and the empty sequence.
"""
import numpy as np
import pytest

import oracle


def _rand(seed, d_conv, d_inner, n_t, n_s):
    rng = np.random.default_rng(seed)
    length = d_conv - 1 + n_t
    sx = rng.uniform(-1, 1, (n_s, d_inner, length))
    w = rng.uniform(-1, 1, (d_inner, d_conv))
    g = rng.uniform(-1, 1, (n_s, n_t, d_inner))
    return sx, w, g


def _loss(sx, w, g, silu):
    return float(np.sum(oracle.conv_fwd(sx, w, apply_silu=silu) * g))


def _central(f, p, eps=1e-5):
    out = np.zeros_like(p)
    flat, grad = p.reshape(-1), out.reshape(-1)
    for k in range(flat.size):
        keep = flat[k]
        flat[k] = keep + eps
        hi = f()
        flat[k] = keep - eps
        lo = f()
        flat[k] = keep
        grad[k] = (hi - lo) / (2 * eps)
    return out


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("d_conv,d_inner,n_t,n_s", [(3, 2, 4, 2), (4, 3, 5, 1), (1, 2, 3, 2)])
def test_conv_bwd_matches_central_difference(silu, d_conv, d_inner, n_t, n_s):
    sx, w, g = _rand(11, d_conv, d_inner, n_t, n_s)
    d_sx, d_w = oracle.conv_bwd(sx, w, g, apply_silu=silu)
    assert d_sx.size + d_w.size == sx.size + w.size
    n_sx = _central(lambda: _loss(sx, w, g, silu), sx)
    n_w = _central(lambda: _loss(sx, w, g, silu), w)
    np.testing.assert_allclose(d_sx, n_sx, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(d_w, n_w, rtol=1e-7, atol=1e-9)


def test_conv_bwd_sum_loss_weight_gradient_is_tap_sum():
    d_conv, d_inner, n_t, n_s = 3, 2, 4, 2
    sx, w, _ = _rand(5, d_conv, d_inner, n_t, n_s)
    g = np.ones((n_s, n_t, d_inner))
    _, d_w = oracle.conv_bwd(sx, w, g)
    ref = np.zeros((d_inner, d_conv))
    for ch in range(d_inner):
        for j in range(d_conv):
            ref[ch, j] = sum(sx[s, ch, t + j] for s in range(n_s) for t in range(n_t))
    np.testing.assert_allclose(d_w, ref, rtol=1e-13, atol=1e-13)


def test_conv_bwd_adjoint_identities():
    sx, w, g = _rand(7, 4, 5, 9, 3)
    d_sx, d_w = oracle.conv_bwd(sx, w, g)
    lhs = _loss(sx, w, g, False)
    assert np.isclose(np.sum(sx * d_sx), lhs, rtol=1e-12, atol=1e-12)
    assert np.isclose(np.sum(w * d_w), lhs, rtol=1e-12, atol=1e-12)


def test_conv_bwd_silu_factor_half_at_zero():
    # w = 0 gives z = 0 everywhere, where d/dz (z s(z)) = 1/2: d_sx = 0 and
    # d_w[j] = sum of g_t sx[t+j] / 2
    sx, _, g = _rand(3, 4, 3, 6, 2)
    w = np.zeros((3, 4))
    d_sx, d_w = oracle.conv_bwd(sx, w, g, apply_silu=True)
    assert not d_sx.any()
    ref = np.zeros_like(w)
    for ch in range(3):
        for j in range(4):
            ref[ch, j] = 0.5 * sum(g[s, t, ch] * sx[s, ch, t + j] for s in range(2) for t in range(6))
    np.testing.assert_allclose(d_w, ref, rtol=1e-13, atol=1e-13)


def test_conv_bwd_no_tokens_gives_zeros():
    sx = np.random.default_rng(0).uniform(-1, 1, (2, 3, 3))  # d_conv 4, n_t 0
    w = np.ones((3, 4))
    d_sx, d_w = oracle.conv_bwd(sx, w, np.zeros((2, 0, 3)))
    assert d_sx.shape == sx.shape and not d_sx.any() and not d_w.any()
