"""Pins for the oracle's GeLU and the feed-forward block chain.

GeLU is checked against scipy's independent normal CDF, exact identities and
finite differences.  The block's backward (unrounded variant) is checked
against central finite differences of the scalar <Y, dY>, which pins the chain
rule, the GeLU derivative and every transpose; the rounded variant is checked
for its rounding points and against its sampled form.
"""
import numpy as np
import pytest
from scipy import special

import oracle
from offload_memory_centric_amd import inputs


def test_gelu_values_and_identities():
    x = np.linspace(-9, 9, 20001)
    g = oracle.gelu(x)
    np.testing.assert_allclose(g, x * special.ndtr(x), rtol=1e-13, atol=1e-300)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(g - oracle.gelu(-x), x, rtol=1e-14, atol=1e-14)
    assert abs(oracle.gelu(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(oracle.gelu(np.array([-30.0]))[0]) < 1e-12


def test_gelu_grad_identities_and_differences():
    assert oracle.gelu_grad(np.array([0.0]))[0] == 0.5
    x = np.linspace(-8, 8, 1601)
    h = 1e-5
    fd = (oracle.gelu(x + h) - oracle.gelu(x - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(x), fd, rtol=0, atol=1e-9)
    # GeLU'(x) + GeLU'(-x) = 1 (derivative of GeLU(x) - GeLU(-x) = x)
    np.testing.assert_allclose(oracle.gelu_grad(x) + oracle.gelu_grad(-x), 1.0, atol=1e-14)


def _ffn_numpy_forward(x, w1, w2):
    """Independent forward with numpy products and scipy's CDF: Y = GeLU(X W1) W2."""
    a = x @ w1
    return (a * special.ndtr(a)) @ w2


def test_ffn_backward_matches_finite_differences():
    T, D, F, D2 = 3, 5, 7, 4
    X = inputs.bits(inputs.new((T, D), "f16", "gaussian", 10, "X"))
    W1t = inputs.bits(inputs.new((F, D), "f16", "gaussian", 10, "W1", std=0.5))
    W2t = inputs.bits(inputs.new((D2, F), "f16", "gaussian", 10, "W2", std=0.5))
    dY = inputs.bits(inputs.new((T, D2), "f16", "gaussian", 10, "dY"))
    x, w1, w2, dy = (oracle.decode(a, "f16") for a in (X, W1t.T.copy(), W2t.T.copy(), dY))
    # forward agrees with the independent composition
    r = oracle.ffn_fwd_bwd(X, W1t, W2t, dY, "f16", round_intermediates=False)
    np.testing.assert_allclose(r["Y"], _ffn_numpy_forward(x, w1, w2), rtol=1e-12, atol=1e-13)

    def loss(x_, w1_, w2_):
        return float((_ffn_numpy_forward(x_, w1_, w2_) * dy).sum())

    h = 1e-6
    for name, arr, grad in (("X", x, r["dX"]), ("W1", w1, r["dW1t"].T), ("W2", w2, r["dW2t"].T)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy()
            p[idx] += h
            m = arr.copy()
            m[idx] -= h
            if name == "X":
                fd[idx] = (loss(p, w1, w2) - loss(m, w1, w2)) / (2 * h)
            elif name == "W1":
                fd[idx] = (loss(x, p, w2) - loss(x, m, w2)) / (2 * h)
            else:
                fd[idx] = (loss(x, w1, p) - loss(x, w1, m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_ffn_rounding_points():
    T, D, F, D2 = 6, 16, 24, 8
    X = inputs.bits(inputs.new((T, D), "f16", "gaussian", 11, "X"))
    W1t = inputs.bits(inputs.new((F, D), "f16", "gaussian", 11, "W1", std=0.3))
    W2t = inputs.bits(inputs.new((D2, F), "f16", "gaussian", 11, "W2", std=0.3))
    dY = inputs.bits(inputs.new((T, D2), "f16", "gaussian", 11, "dY"))
    r = oracle.ffn_fwd_bwd(X, W1t, W2t, dY, "f16")
    u = oracle.ffn_fwd_bwd(X, W1t, W2t, dY, "f16", round_intermediates=False)
    # A and H are fp16 values: A is the RNE of the exact product, H the RNE of GeLU(A)
    assert np.array_equal(r["A"], oracle.round_to(u["A"], "f16"))
    assert np.array_equal(r["H"], oracle.round_to(oracle.gelu(r["A"]), "f16"))
    # dA = RNE(dH * GeLU'(A)) with dH unrounded
    assert np.array_equal(r["dA"], oracle.round_to(r["dH"] * oracle.gelu_grad(r["A"]), "f16"))
    # the rounded chain stays close to the unrounded one
    for k in ("Y", "dX", "dW1t", "dW2t"):
        assert np.abs(r[k] - u[k]).max() <= 2e-2 * np.abs(u[k]).max() + 1e-12, k


def test_ffn_sample_equals_full():
    T, D, F, D2 = 10, 24, 40, 16
    X = inputs.bits(inputs.new((T, D), "f16", "gaussian", 12, "X"))
    W1t = inputs.bits(inputs.new((F, D), "f16", "gaussian", 12, "W1", std=0.2))
    W2t = inputs.bits(inputs.new((D2, F), "f16", "gaussian", 12, "W2", std=0.2))
    dY = inputs.bits(inputs.new((T, D2), "f16", "gaussian", 12, "dY"))
    full = oracle.ffn_fwd_bwd(X, W1t, W2t, dY, "f16")
    tr, fc, d2c, dc = [0, 3, 9], [0, 17, 39], [1, 15], [0, 23]
    s = oracle.ffn_sample(X, W1t, W2t, dY, "f16", tr, fc, d2c, dc, chunk=7)
    assert np.array_equal(s["A"], full["A"][np.ix_(tr, fc)])
    assert np.array_equal(s["H"], full["H"][np.ix_(tr, fc)])
    assert np.array_equal(s["Y"], full["Y"][np.ix_(tr, d2c)])
    assert np.array_equal(s["dH"], full["dH"][np.ix_(tr, fc)])
    assert np.array_equal(s["dA"], full["dA"][np.ix_(tr, fc)])
    assert np.array_equal(s["dX"], full["dX"][np.ix_(tr, dc)])
    assert np.array_equal(s["dW1t"], full["dW1t"][np.ix_(fc, dc)])
    assert np.array_equal(s["dW2t"], full["dW2t"][np.ix_(d2c, fc)])
