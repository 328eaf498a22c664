"""CPU oracle for memory-centric tiling of a large linear operator Y = XW.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``offload_memory_centric_amd``) and never imports it; the
GPU library never imports this package.

What it computes, untiled and in double precision (the pages fix no precision
for a checker, so every sum is carried in fp64; fp16/bf16 inputs decode into
double exactly):

* ``linear_fwd``   Y = X W.  The memory-centric tiling method (ZeRO-Infinity
  transformer-math page, section "Memory-centric tiling: operators bigger than
  the device"; pwwt.cn ZeRO-Infinity article, section
  "关键技术一：Memory-centric tiling", core idea) splits W along its output
  dimension, computes each slice X W_i and concatenates the slices.  Splitting
  the columns of a product and concatenating is exactly the product, so the
  oracle is the plain untiled definition.
* ``linear_bwd``   dX = dY W^T and dW = X^T dY, the two products of the
  backward pass that the FLOPs-per-byte section of the transformer-math page
  counts as 4P per token.
* ``ffn_fwd_bwd``  the feed-forward block that section's 1T-model example
  names (25600 -> 102400 -> 25600): A = X W1, H = GeLU(A), Y = H W2, then the
  backward with the GeLU derivative.  A, H and dA are stored by the method in
  the 16-bit input format, so the oracle rounds them there (RNE) too.

* ``adam_step``    the optimizer step that runs beside the path: the
  transformer-math page (section "Applying the test: which state can live
  where", its remark on the Adam update) puts it on the CPU because it is
  elementwise (ait about 0.5); the GPU ZeRO-sharding page (section "The
  architecture: every piece explained", the state taxonomy and offload) gives
  its state as an fp32 master weight and first and second moments, and its
  section "End-to-end flow" has the updated 16-bit parameters become the next
  step's resting copy.  The update itself is Adam as Kingma and Ba publish it
  (bias-corrected moments, no weight decay), in double precision.

Host layout of a weight: out-major, W^t[M x K] (row m holds column m of W), the
layout of ``nn.Linear.weight``; tile i is then rows [i*n, (i+1)*n) of W^t.

Parity pins for all of this live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "zio.c")

DTYPES = {"f16": 1, "bf16": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile zio.c with gcc into oracle/liboracle.so (IEEE order kept:
    no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               "-fno-fast-math", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.zio_decode1.argtypes = [ctypes.c_int, ctypes.c_uint16]
    lib.zio_decode1.restype = ctypes.c_double
    lib.zio_encode1.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.zio_encode1.restype = ctypes.c_uint16
    lib.zio_decode.argtypes = [ctypes.c_int, p, i64, p]
    lib.zio_encode.argtypes = [ctypes.c_int, p, i64, p]
    lib.zio_gather.argtypes = [ctypes.c_int, p, i64, i64, i64, p, i64, p, p]
    lib.zio_matmul_nt.argtypes = [i64, i64, i64, p, p, p]
    lib.zio_gelu.argtypes = [p, i64, p]
    lib.zio_gelu.restype = None
    lib.zio_gelu_grad.argtypes = [p, i64, p]
    lib.zio_gelu_grad.restype = None
    lib.zio_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def set_threads(n: int = 0) -> int:
    """Threads used by the oracle (0 = every core this process may run on)."""
    return _load().zio_set_threads(int(n))


def get_threads() -> int:
    return _load().zio_get_threads()


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dt(dtype: str) -> int:
    if dtype not in DTYPES:
        raise ValueError("dtype must be 'f16' or 'bf16'")
    return DTYPES[dtype]


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("16-bit operands are passed as their uint16 bit patterns")
    return a


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def decode(bits, dtype: str) -> np.ndarray:
    """Exact double value of each binary16 / bfloat16 bit pattern."""
    b = np.ascontiguousarray(_u16(bits))
    out = np.empty(b.shape, dtype=np.float64)
    if _load().zio_decode(_dt(dtype), _ptr(b), b.size, _ptr(out)) != 0:
        raise ValueError("decode failed")
    return out


def encode(x, dtype: str) -> np.ndarray:
    """Round-to-nearest-even encoding of doubles into the 16-bit format."""
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    if _load().zio_encode(_dt(dtype), _ptr(v), v.size, _ptr(out)) != 0:
        raise ValueError("encode failed")
    return out


def round_to(x, dtype: str) -> np.ndarray:
    """Value after one RNE rounding into the 16-bit format."""
    return decode(encode(x, dtype), dtype)


def gather(bits, dtype: str, row_stride: int, col_stride: int,
           rows: Optional[Sequence[int]], nrows: int,
           cols: Optional[Sequence[int]], ncols: int) -> np.ndarray:
    """Decoded dense copy  out[r][c] = value(bits.flat[rows[r]*row_stride + cols[c]*col_stride]).

    ``rows``/``cols`` = None means 0..nrows-1 / 0..ncols-1.  ``bits`` may be any
    C-contiguous uint16 array (a pinned host tensor's memory, for instance)."""
    b = _u16(bits)
    if not b.flags["C_CONTIGUOUS"]:
        raise ValueError("gather needs a C-contiguous source")
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = None if cols is None else np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    nr = nrows if r is None else r.size
    nc = ncols if c is None else c.size
    # bounds of every element that will be read
    hi = 0
    if nr and nc:
        rmax = (nrows - 1) if r is None else int(r.max())
        cmax = (ncols - 1) if c is None else int(c.max())
        rmin = 0 if r is None else int(r.min())
        cmin = 0 if c is None else int(c.min())
        if rmin < 0 or cmin < 0:
            raise IndexError("negative index")
        hi = rmax * row_stride + cmax * col_stride
        if hi >= b.size:
            raise IndexError("gather reads past the source")
    out = np.empty((nr, nc), dtype=np.float64)
    rc = _load().zio_gather(_dt(dtype), _ptr(b), row_stride, col_stride,
                            nr, None if r is None else _ptr(r),
                            nc, None if c is None else _ptr(c), _ptr(out))
    if rc != 0:
        raise ValueError("gather failed")
    return out


def matmul_nt(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C[r][c] = sum_i A[r][i] * B[c][i] in double, each sum in ascending i."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("matmul_nt: shapes %s, %s" % (A.shape, B.shape))
    C = np.empty((A.shape[0], B.shape[0]), dtype=np.float64)
    if _load().zio_matmul_nt(A.shape[0], B.shape[0], A.shape[1], _ptr(A), _ptr(B), _ptr(C)) != 0:
        raise ValueError("matmul_nt failed")
    return C


def gelu(a) -> np.ndarray:
    """GeLU(a) = a * Phi(a) with the exact erf form of the normal CDF."""
    v = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    out = np.empty_like(v)
    _load().zio_gelu(_ptr(v), v.size, _ptr(out))
    return out


def gelu_grad(a) -> np.ndarray:
    """GeLU'(a) = Phi(a) + a * phi(a)."""
    v = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    out = np.empty_like(v)
    _load().zio_gelu_grad(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# the linear operator, untiled
# ---------------------------------------------------------------------------

def _shape2(a, name):
    a = _u16(a)
    if a.ndim != 2:
        raise ValueError("%s must be 2-D" % name)
    return a


def linear_fwd(X, Wt, dtype: str) -> np.ndarray:
    """Y[t][m] = sum_k X[t][k] * W[k][m], with W[k][m] = Wt[m][k].  Returns fp64 [T x M]."""
    X, Wt = _shape2(X, "X"), _shape2(Wt, "Wt")
    T, K = X.shape
    M = Wt.shape[0]
    if Wt.shape[1] != K:
        raise ValueError("inner dimensions differ")
    Xd = gather(np.ascontiguousarray(X), dtype, K, 1, None, T, None, K)
    Wd = gather(np.ascontiguousarray(Wt), dtype, K, 1, None, M, None, K)   # row m = column m of W
    return matmul_nt(Xd, Wd)


def linear_bwd(X, Wt, dY, dtype: str):
    """Backward of Y = XW for an upstream gradient dY[T x M].

    dX[t][k]  = sum_m dY[t][m] * W[k][m]
    dWt[m][k] = dW[k][m] = sum_t X[t][k] * dY[t][m]   (returned out-major, like Wt)
    Both fp64."""
    X, Wt, dY = _shape2(X, "X"), _shape2(Wt, "Wt"), _shape2(dY, "dY")
    T, K = X.shape
    M = Wt.shape[0]
    if Wt.shape[1] != K or dY.shape != (T, M):
        raise ValueError("shapes disagree")
    X, Wt, dY = (np.ascontiguousarray(a) for a in (X, Wt, dY))
    dYd = gather(dY, dtype, M, 1, None, T, None, M)          # [T x M]
    Wd_T = gather(Wt, dtype, 1, K, None, K, None, M)         # [K x M]: row k = row k of W
    dX = matmul_nt(dYd, Wd_T)
    dYd_T = gather(dY, dtype, 1, M, None, M, None, T)        # [M x T]
    Xd_T = gather(X, dtype, 1, K, None, K, None, T)          # [K x T]
    dWt = matmul_nt(dYd_T, Xd_T)                             # [M x K]
    return dX, dWt


# sampled entries, for shapes too large to compute whole --------------------

def linear_fwd_sample(X, Wt, rows, cols, dtype: str) -> np.ndarray:
    """Y[rows][:, cols] of Y = XW, each entry a full-length dot product."""
    T, K = X.shape
    M = Wt.shape[0]
    Xd = gather(X, dtype, K, 1, rows, T, None, K)
    Wd = gather(Wt, dtype, K, 1, cols, M, None, K)
    return matmul_nt(Xd, Wd)


def linear_dx_sample(Wt, dY, rows, cols, dtype: str) -> np.ndarray:
    """dX[rows][:, cols] with dX = dY W^T."""
    T, M = dY.shape
    K = Wt.shape[1]
    dYd = gather(dY, dtype, M, 1, rows, T, None, M)
    Wd_T = gather(Wt, dtype, 1, K, cols, K, None, M)
    return matmul_nt(dYd, Wd_T)


def linear_dw_sample(X, dY, mrows, kcols, dtype: str) -> np.ndarray:
    """dWt[mrows][:, kcols] (out-major gradient) with dW = X^T dY."""
    T, K = X.shape
    M = dY.shape[1]
    dYd_T = gather(dY, dtype, 1, M, mrows, M, None, T)
    Xd_T = gather(X, dtype, 1, K, kcols, K, None, T)
    return matmul_nt(dYd_T, Xd_T)


# ---------------------------------------------------------------------------
# the feed-forward block: up-projection, GeLU, down-projection
# ---------------------------------------------------------------------------

def ffn_fwd_bwd(X, W1t, W2t, dY, dtype: str, round_intermediates: bool = True) -> Dict[str, np.ndarray]:
    """Forward and backward of Y = GeLU(X W1) W2 for upstream gradient dY.

    Shapes: X [T x D], W1t [F x D] (W1 is D x F), W2t [D2 x F] (W2 is F x D2),
    dY [T x D2].  With ``round_intermediates`` the stored activations A, H and
    the stored gradient dA are rounded once (RNE) into ``dtype``, as the method
    stores them; dH stays unrounded (it is accumulated in fp32 across tiles).
    Returns A, H (rounded values), Y, dH, dA (rounded), dX, dW1t, dW2t (fp64),
    and the two quantities the method rounds before storing them, unrounded:
    A_exact = X W1 and dA_exact = dH * GeLU'(A) (with A the rounded value).
    """
    T, D = X.shape
    F = W1t.shape[0]
    D2 = W2t.shape[0]
    A = linear_fwd(X, W1t, dtype)
    A_r = round_to(A, dtype) if round_intermediates else A
    H = gelu(A_r)
    H_r = round_to(H, dtype) if round_intermediates else H
    H_bits = encode(H_r, dtype) if round_intermediates else None
    if round_intermediates:
        Y = linear_fwd(H_bits, W2t, dtype)
        dH, dW2t = linear_bwd(H_bits, W2t, dY, dtype)
    else:
        W2d = gather(np.ascontiguousarray(W2t), dtype, F, 1, None, D2, None, F)  # [D2 x F]
        Y = matmul_nt(H_r, W2d)
        dYd = gather(np.ascontiguousarray(dY), dtype, D2, 1, None, T, None, D2)
        dH = matmul_nt(dYd, np.ascontiguousarray(W2d.T))
        dW2t = matmul_nt(np.ascontiguousarray(dYd.T), np.ascontiguousarray(H_r.T))
    dA = dH * gelu_grad(A_r)
    dA_r = round_to(dA, dtype) if round_intermediates else dA
    if round_intermediates:
        dA_bits = encode(dA_r, dtype)
        dX, dW1t = linear_bwd(X, W1t, dA_bits, dtype)
    else:
        W1d_T = gather(np.ascontiguousarray(W1t), dtype, 1, D, None, D, None, F)  # [D x F]
        Xd = gather(np.ascontiguousarray(X), dtype, D, 1, None, T, None, D)
        dX = matmul_nt(dA_r, W1d_T)
        dW1t = matmul_nt(np.ascontiguousarray(dA_r.T), np.ascontiguousarray(Xd.T))
    return {"A": A_r, "H": H_r, "Y": Y, "dH": dH, "dA": dA_r,
            "dX": dX, "dW1t": dW1t, "dW2t": dW2t, "A_exact": A, "dA_exact": dA}


def ffn_sample(X, W1t, W2t, dY, dtype: str, t_rows, f_cols, d2_cols, d_cols,
               chunk: int = 2048) -> Dict[str, np.ndarray]:
    """Sampled entries of every output of ``ffn_fwd_bwd`` (rounded intermediates).

    t_rows: token rows; f_cols: hidden (F) columns; d2_cols: output (D2)
    columns; d_cols: input (D) columns.  Returns
      A[t_rows][:, f_cols], H[...], Y[t_rows][:, d2_cols], dH[t_rows][:, f_cols],
      dA[t_rows][:, f_cols], dX[t_rows][:, d_cols],
      dW1t[f_cols][:, d_cols], dW2t[d2_cols][:, f_cols].
    Each entry follows the same chain as ``ffn_fwd_bwd``; the full-length
    rows / columns an entry depends on are computed whole, in chunks of the
    hidden dimension to bound memory.
    """
    T, D = X.shape
    F = W1t.shape[0]
    D2 = W2t.shape[0]
    t_rows = np.asarray(t_rows, dtype=np.int64)
    f_cols = np.asarray(f_cols, dtype=np.int64)
    nt = t_rows.size

    # rows t of A, H, dH, dA over the whole hidden dimension
    Xr = gather(X, dtype, D, 1, t_rows, T, None, D)                 # [nt x D]
    dYr = gather(dY, dtype, D2, 1, t_rows, T, None, D2)             # [nt x D2]
    A_rows = np.empty((nt, F))
    dH_rows = np.empty((nt, F))
    for f0 in range(0, F, chunk):
        f1 = min(F, f0 + chunk)
        fidx = np.arange(f0, f1, dtype=np.int64)
        W1c = gather(W1t, dtype, D, 1, fidx, F, None, D)            # [c x D]: W1[:, f]
        A_rows[:, f0:f1] = matmul_nt(Xr, W1c)
        W2c_T = gather(W2t, dtype, 1, F, fidx, F, None, D2)         # [c x D2]: W2[f, :]
        dH_rows[:, f0:f1] = matmul_nt(dYr, W2c_T)
    A_rows = round_to(A_rows, dtype)
    H_rows = round_to(gelu(A_rows), dtype)
    dA_rows = round_to(dH_rows * gelu_grad(A_rows), dtype)

    # Y rows: H[t, :] W2[:, d2]
    W2s = gather(W2t, dtype, F, 1, d2_cols, D2, None, F)            # [n2 x F]
    Y_s = matmul_nt(H_rows, W2s)
    # dX rows: dA[t, :] W1[d, :]^T  (W1[d][f] = W1t[f][d])
    W1s_T = gather(W1t, dtype, 1, D, d_cols, D, None, F)            # [nd x F]
    dX_s = matmul_nt(dA_rows, W1s_T)

    # columns f of A, H, dH, dA over all tokens
    W1f = gather(W1t, dtype, D, 1, f_cols, F, None, D)              # [nf x D]
    W2f_T = gather(W2t, dtype, 1, F, f_cols, F, None, D2)           # [nf x D2]
    A_cols = np.empty((T, f_cols.size))
    dH_cols = np.empty((T, f_cols.size))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        tidx = np.arange(t0, t1, dtype=np.int64)
        Xc = gather(X, dtype, D, 1, tidx, T, None, D)
        dYc = gather(dY, dtype, D2, 1, tidx, T, None, D2)
        A_cols[t0:t1] = matmul_nt(Xc, W1f)
        dH_cols[t0:t1] = matmul_nt(dYc, W2f_T)
    A_cols = round_to(A_cols, dtype)
    H_cols = round_to(gelu(A_cols), dtype)
    dA_cols = round_to(dH_cols * gelu_grad(A_cols), dtype)
    # dW2t[d2][f] = sum_t H[t][f] dY[t][d2]
    dY_T = gather(dY, dtype, 1, D2, d2_cols, D2, None, T)           # [n2 x T]
    dW2t_s = matmul_nt(dY_T, np.ascontiguousarray(H_cols.T))
    # dW1t[f][d] = sum_t dA[t][f] X[t][d]
    X_T = gather(X, dtype, 1, D, d_cols, D, None, T)                # [nd x T]
    dW1t_s = matmul_nt(np.ascontiguousarray(dA_cols.T), X_T)
    return {"A": A_rows[:, f_cols], "H": H_rows[:, f_cols], "Y": Y_s,
            "dH": dH_rows[:, f_cols], "dA": dA_rows[:, f_cols], "dX": dX_s,
            "dW1t": dW1t_s, "dW2t": dW2t_s,
            "A_cols": A_cols, "dA_cols": dA_cols}


def adam_step(master, m, v, grad, step: int, lr: float, beta1: float, beta2: float, eps: float):
    """One Adam step (Kingma and Ba: bias-corrected first and second moments,
    no weight decay) in double precision; returns (master, m, v) after step
    `step` (1 for the first).  grad is the gradient of this step (dW)."""
    if step < 1:
        raise ValueError("step counts from 1")
    master = np.asarray(master, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    m1 = beta1 * m + (1.0 - beta1) * g
    v1 = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m1 / (1.0 - beta1 ** step)
    v_hat = v1 / (1.0 - beta2 ** step)
    return master - lr * m_hat / (np.sqrt(v_hat) + eps), m1, v1
