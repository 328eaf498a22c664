"""Pins for the oracle's untiled linear operator and its adjoints.

Each check uses something other than the oracle itself: pure-Python loops on
tiny shapes, numpy's float64 BLAS product, the adjoint identity in exact
integer arithmetic, one-hot and ramp inputs whose results are known in closed
form, and agreement of the sampled entry points with the full ones.
"""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs


def _gauss(shape, seed, tid, std=1.0, dtype="f16"):
    return inputs.bits(inputs.new(shape, dtype, "gaussian", seed, tid, std=std))


def _ints(shape, seed, tid, dtype="f16"):
    return inputs.bits(inputs.new(shape, dtype, "small_int", seed, tid))


def _val(bits, dtype="f16"):
    return oracle.decode(bits, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fwd_bwd_equal_python_loops(dtype):
    T, K, M = 3, 5, 4
    X, Wt, dY = _gauss((T, K), 0, "X", dtype=dtype), _gauss((M, K), 0, "W", 0.5, dtype), _gauss((T, M), 0, "dY", dtype=dtype)
    x, w, dy = _val(X, dtype), _val(Wt, dtype), _val(dY, dtype)
    Y = oracle.linear_fwd(X, Wt, dtype)
    dX, dWt = oracle.linear_bwd(X, Wt, dY, dtype)
    for t in range(T):
        for m in range(M):
            s = 0.0
            for k in range(K):
                s += x[t][k] * w[m][k]          # W[k][m] = Wt[m][k]
            assert Y[t][m] == s
    for t in range(T):
        for k in range(K):
            s = 0.0
            for m in range(M):
                s += dy[t][m] * w[m][k]
            assert dX[t][k] == s
    for m in range(M):
        for k in range(K):
            s = 0.0
            for t in range(T):
                s += x[t][k] * dy[t][m]
            assert dWt[m][k] == s


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_against_numpy_blas(dtype):
    T, K, M = 37, 72, 48
    X, Wt, dY = _gauss((T, K), 1, "X", dtype=dtype), _gauss((M, K), 1, "W", 0.02, dtype), _gauss((T, M), 1, "dY", dtype=dtype)
    x, w, dy = _val(X, dtype), _val(Wt, dtype), _val(dY, dtype)
    W = w.T                                            # logical W[K x M]
    Y = oracle.linear_fwd(X, Wt, dtype)
    dX, dWt = oracle.linear_bwd(X, Wt, dY, dtype)
    np.testing.assert_allclose(Y, x @ W, rtol=1e-12, atol=1e-12 * np.abs(x @ W).max())
    np.testing.assert_allclose(dX, dy @ W.T, rtol=1e-12, atol=1e-12 * np.abs(dX).max())
    np.testing.assert_allclose(dWt, (x.T @ dy).T, rtol=1e-12, atol=1e-12 * np.abs(dWt).max())
    assert Y.shape == (T, M) and dX.shape == (T, K) and dWt.shape == (M, K)


def test_adjoint_identity_exact_integers():
    # <Y, dY> = <X, dX> = <W, dW> = tr(W^T X^T dY), exact for small integers
    T, K, M = 16, 40, 24
    X, Wt, dY = _ints((T, K), 2, "X"), _ints((M, K), 2, "W"), _ints((T, M), 2, "dY")
    Y = oracle.linear_fwd(X, Wt, "f16")
    dX, dWt = oracle.linear_bwd(X, Wt, dY, "f16")
    xi, wi, dyi = (_val(a).astype(np.int64) for a in (X, Wt, dY))
    Yi, dXi, dWi = (a.astype(np.int64) for a in (Y, dX, dWt))
    assert np.array_equal(Yi, Y) and np.array_equal(dXi, dX) and np.array_equal(dWi, dWt)
    a = int((Yi * dyi).sum())
    b = int((xi * dXi).sum())
    c = int((wi * dWi).sum())
    assert a == b == c
    # and the integer product itself, computed with exact integer matmul
    assert np.array_equal(Yi, xi @ wi.T)


def test_one_hot_inputs():
    K, M = 12, 10
    Wt = _gauss((M, K), 3, "W", 0.3)
    w = _val(Wt)
    eye = np.eye(K)
    X = oracle.encode(eye, "f16")                       # X = I -> Y = W
    Y = oracle.linear_fwd(X, Wt, "f16")
    assert np.array_equal(Y, w.T)
    # one-hot upstream gradient: dY[t] = e_j
    j, t0 = 7, 4
    dy = np.zeros((K, M))
    dy[t0, j] = 1.0
    dX, dWt = oracle.linear_bwd(X, Wt, oracle.encode(dy, "f16"), "f16")
    expect_dx = np.zeros((K, K))
    expect_dx[t0] = w[j]                                # row j of W^t = column j of W
    assert np.array_equal(dX, expect_dx)
    expect_dw = np.zeros((M, K))
    expect_dw[j, t0] = 1.0                              # outer product x_t0 (= e_t0) with e_j
    assert np.array_equal(dWt, expect_dw)


def test_ramp_exposes_column_offsets():
    # X = e_0 rows, W[0][m] = m mod 2048 (exact in fp16): Y[t][m] = m mod 2048
    T, K, M = 8, 16, 4096
    x = np.zeros((T, K))
    x[:, 0] = 1.0
    w = np.zeros((M, K))
    w[:, 0] = np.arange(M) % 2048
    Y = oracle.linear_fwd(oracle.encode(x, "f16"), oracle.encode(w, "f16"), "f16")
    assert np.array_equal(Y, np.tile(np.arange(M) % 2048, (T, 1)).astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_sampled_entries_equal_full(dtype):
    T, K, M = 40, 64, 96
    X, Wt, dY = _gauss((T, K), 4, "X", dtype=dtype), _gauss((M, K), 4, "W", 0.02, dtype), _gauss((T, M), 4, "dY", dtype=dtype)
    Y = oracle.linear_fwd(X, Wt, dtype)
    dX, dWt = oracle.linear_bwd(X, Wt, dY, dtype)
    rows, cols, kc = [0, 5, 39], [0, 31, 32, 95], [0, 1, 63]
    assert np.array_equal(oracle.linear_fwd_sample(X, Wt, rows, cols, dtype), Y[np.ix_(rows, cols)])
    assert np.array_equal(oracle.linear_dx_sample(Wt, dY, rows, kc, dtype), dX[np.ix_(rows, kc)])
    assert np.array_equal(oracle.linear_dw_sample(X, dY, cols, kc, dtype), dWt[np.ix_(cols, kc)])


def test_column_split_concatenation_is_the_product():
    # The method's own statement: Y = [X W_1, ..., X W_N].  Concatenating the
    # oracle's products of the column slices reproduces the untiled product
    # bit for bit (each entry is the same dot product).
    T, K, M, N = 9, 32, 48, 4
    n = M // N
    X, Wt = _gauss((T, K), 5, "X"), _gauss((M, K), 5, "W", 0.02)
    Y = oracle.linear_fwd(X, Wt, "f16")
    parts = [oracle.linear_fwd(X, np.ascontiguousarray(Wt[i * n:(i + 1) * n]), "f16") for i in range(N)]
    assert np.array_equal(np.concatenate(parts, axis=1), Y)


def test_thread_count_does_not_change_results():
    T, K, M = 33, 64, 40
    X, Wt, dY = _gauss((T, K), 6, "X"), _gauss((M, K), 6, "W", 0.02), _gauss((T, M), 6, "dY")
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = oracle.linear_bwd(X, Wt, dY, "f16")
        oracle.set_threads(5)
        b = oracle.linear_bwd(X, Wt, dY, "f16")
    finally:
        oracle.set_threads(old)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rounded_outputs_single_rne():
    # The stored fp16 output is one RNE rounding of the exact sum: for small
    # integers the sum is exact, so the stored value is numpy's rounding of it.
    T, K, M = 8, 512, 64
    X, Wt = _ints((T, K), 7, "X"), _ints((M, K), 7, "W")
    Y = oracle.linear_fwd(X, Wt, "f16")
    assert np.array_equal(oracle.encode(Y, "f16"), Y.astype(np.float16).view(np.uint16))
