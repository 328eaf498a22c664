"""Pins of the oracle's Adam step (oracle.adam_step) against closed forms of
the published algorithm (Kingma and Ba), independent of its code path."""
import numpy as np
import pytest

import oracle

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def test_first_step_is_a_signed_unit_step():
    # from zero moments, m_hat = g and v_hat = g^2 after one step, so the
    # update is lr * g / (|g| + eps): a step of lr in the direction of -sign(g)
    rng = np.random.default_rng(0)
    w = rng.normal(0, 0.02, 1000)
    g = rng.normal(0, 1e-2, 1000)
    w1, m1, v1 = oracle.adam_step(w, 0 * w, 0 * w, g, 1, LR, B1, B2, EPS)
    assert np.allclose(w1, w - LR * g / (np.abs(g) + EPS), rtol=0, atol=1e-15)
    assert np.allclose(m1, (1 - B1) * g, rtol=1e-15, atol=0)
    assert np.allclose(v1, (1 - B2) * g * g, rtol=1e-15, atol=0)


def test_constant_gradient_moves_linearly():
    # with the same g at every step the bias-corrected moments stay exactly
    # g and g^2, so t steps move the weight by t * lr * g / (|g| + eps)
    g = np.array([3e-3, -2e-1, 5.0, -7e-5])
    w = np.array([0.01, -0.02, 0.03, 0.0])
    m = v = np.zeros_like(w)
    cur = w
    for t in range(1, 51):
        cur, m, v = oracle.adam_step(cur, m, v, g, t, LR, B1, B2, EPS)
    assert np.allclose(cur, w - 50 * LR * g / (np.abs(g) + EPS), rtol=0, atol=1e-12)
    assert np.allclose(m, g * (1 - B1 ** 50), rtol=1e-12, atol=0)
    assert np.allclose(v, g * g * (1 - B2 ** 50), rtol=1e-12, atol=0)


def test_second_step_with_zero_gradient_by_hand():
    # step 1 with g, step 2 with 0: m2 = b1 (1 - b1) g, v2 = b2 (1 - b2) g^2,
    # m_hat = m2 / (1 - b1^2), v_hat = v2 / (1 - b2^2); written out for a scalar
    g, w = 0.25, 0.5
    w1, m1, v1 = oracle.adam_step(np.array([w]), np.zeros(1), np.zeros(1), np.array([g]), 1, LR, B1, B2, EPS)
    w2, m2, v2 = oracle.adam_step(w1, m1, v1, np.zeros(1), 2, LR, B1, B2, EPS)
    mh = B1 * (1 - B1) * g / (1 - B1 * B1)
    vh = B2 * (1 - B2) * g * g / (1 - B2 * B2)
    want = w - LR * g / (abs(g) + EPS) - LR * mh / (np.sqrt(vh) + EPS)
    assert abs(w2[0] - want) <= 1e-15
    assert abs(m2[0] - B1 * (1 - B1) * g) <= 1e-17 and abs(v2[0] - B2 * (1 - B2) * g * g) <= 1e-18


def test_sign_symmetry_and_scale_invariance():
    rng = np.random.default_rng(1)
    w = rng.normal(0, 0.02, 64)
    g1, g2 = rng.normal(0, 1, 64), rng.normal(0, 1, 64)
    a = oracle.adam_step(w, 0 * w, 0 * w, g1, 1, LR, B1, B2, EPS)
    a = oracle.adam_step(a[0], a[1], a[2], g2, 2, LR, B1, B2, EPS)
    b = oracle.adam_step(-w, 0 * w, 0 * w, -g1, 1, LR, B1, B2, EPS)
    b = oracle.adam_step(b[0], b[1], b[2], -g2, 2, LR, B1, B2, EPS)
    assert np.allclose(a[0], -b[0], rtol=0, atol=1e-16)
    # with eps = 0 the update does not depend on the gradient's scale
    c = oracle.adam_step(w, 0 * w, 0 * w, g1, 1, LR, B1, B2, 0.0)
    c = oracle.adam_step(c[0], c[1], c[2], g2, 2, LR, B1, B2, 0.0)
    d = oracle.adam_step(w, 0 * w, 0 * w, 1e3 * g1, 1, LR, B1, B2, 0.0)
    d = oracle.adam_step(d[0], d[1], d[2], 1e3 * g2, 2, LR, B1, B2, 0.0)
    assert np.allclose(c[0], d[0], rtol=0, atol=1e-15)


def test_step_counts_from_one():
    with pytest.raises(ValueError):
        oracle.adam_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), 0, LR, B1, B2, EPS)
