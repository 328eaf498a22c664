"""Shared helpers for the GPU parity tests: build inputs, run the library
through its C ABI, and compare with the oracle.

Expected values come only from ``oracle``; inputs only from
``offload_memory_centric_amd.inputs``.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from offload_memory_centric_amd import inputs

TOL = 2e-3  # max |gpu - ref| <= TOL * max |ref|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def lib():
    """The binding; importing it fails loudly when libzi.so is missing."""
    from offload_memory_centric_amd import tiling, zi  # noqa: F401
    return tiling


def host_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view of a 16-bit tensor's bytes (copied to host if on the GPU)."""
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def values(t: torch.Tensor, dtype: str) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy().astype(np.float64)
    return oracle.decode(host_bits(t), dtype)


def max_err(got: np.ndarray, ref: np.ndarray):
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return err, scale


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    err, scale = max_err(got, ref)
    say("  %-12s max|err| %.3e  max|ref| %.3e  ratio %.2e" % (what, err, scale, err / scale if scale else 0))
    assert err <= tol * scale, "%s: max|err| %.3e > %.1e * max|ref| %.3e" % (what, err, tol, scale)


def ulp(x: float, dtype: str) -> float:
    """Spacing of the 16-bit format at |x| (its binade's unit in the last place)."""
    mant = 10 if dtype == "f16" else 7
    x = abs(float(x))
    if x == 0.0:
        return 0.0
    return 2.0 ** (np.floor(np.log2(x)) - mant)


def stored_tol(ref: np.ndarray, dtype: str, ulps: float) -> float:
    """Relative bound for a value the method stores in 16 bits, compared with
    the oracle's chain.  fp16: the 2e-3 bar (its half-ulp is at most 4.9e-4 of
    the maximum).  bf16: 2e-3 for the fp32 arithmetic plus `ulps` units in the
    last place at max|ref|: 1/2 for the method's own rounding of a value the
    oracle keeps unrounded (Y, dW); 1 where both round the same quantity and
    may take neighbouring values when it lies within the fp32 sum's error of a
    rounding boundary (A); 1 + 1.13 where the input was such a neighbour too
    (H = GeLU(A), |GeLU'| <= 1.13)."""
    if dtype == "f16":
        return TOL
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return TOL + (ulps * ulp(scale, dtype) / scale if scale else 0.0)


def make_linear_inputs(T, K, M, dtype, kind, seed, device="cuda", w_std=0.02, gen_device=None,
                       chunk_rows=0):
    """X [T,K] and dY [T,M] on `device`; W^t [M,K] in pinned host memory."""
    tiling = lib()
    std = 1.0 if kind == "gaussian" else 1.0
    X = inputs.new((T, K), dtype, kind, seed, "X", std=std, device=device)
    dY = inputs.new((T, M), dtype, kind, seed, "dY", std=std, device=device)
    Wt = tiling.host_tensor((M, K), inputs.torch_dtype(dtype))
    inputs.fill_(Wt, kind, seed, "W", std=(w_std if kind == "gaussian" else 1.0),
                 device=gen_device or device, chunk_rows=chunk_rows)
    return X, Wt, dY


def sample_indices(extent: int, count: int, seed: int, must=()):
    rng = np.random.default_rng(seed)
    idx = set(int(i) for i in must if 0 <= i < extent)
    idx.update(int(i) for i in rng.choice(extent, size=min(count, extent), replace=False))
    idx.update({0, extent - 1})
    return np.array(sorted(idx), dtype=np.int64)


def tile_edges(M: int, n: int):
    e = []
    for i in range(1, M // n):
        e += [i * n - 1, i * n]
    return e
