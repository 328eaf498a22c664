"""GPU parity of the feed-forward block (up-projection, GeLU, down-projection)
with activation checkpointing, against the oracle's chain (small shapes)."""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import assert_close, host_bits, lib, say, values

pytestmark = pytest.mark.gpu


def ffn_setup(T, D, F, N1, N2, d, dtype, seed, w_std=0.02):
    tiling = lib()
    tdt = inputs.torch_dtype(dtype)
    X = inputs.new((T, D), dtype, "gaussian", seed, "X", device="cuda")
    dY = inputs.new((T, D), dtype, "gaussian", seed, "dY", device="cuda")
    W1t = tiling.host_tensor((F, D), tdt)          # W1 [D x F], out-major
    W2t = tiling.host_tensor((D, F), tdt)          # W2 [F x D], out-major
    inputs.fill_(W1t, "gaussian", seed, "W1", std=w_std, device="cuda")
    inputs.fill_(W2t, "gaussian", seed, "W2", std=w_std, device="cuda")
    dW1t = tiling.host_tensor((F, D), tdt)
    dW2t = tiling.host_tensor((D, F), tdt)
    p1 = tiling.Plan(T, D, F, N1, d, dtype, W1t, dW1t)
    p2 = tiling.Plan(T, F, D, N2, d, dtype, W2t, dW2t)
    # one ring for both operators: the slots fit the larger tile of the two
    big = p1 if p1.info.ring_bytes >= p2.info.ring_bytes else p2
    ctx = tiling.Context(big)
    bufs = {
        "X": X, "dY": dY,
        "A": torch.empty((T, F), dtype=tdt, device="cuda"),
        "H": torch.empty((T, F), dtype=tdt, device="cuda"),
        "Y": torch.empty((T, D), dtype=tdt, device="cuda"),
        "Yr": torch.empty((T, D), dtype=tdt, device="cuda"),
        "dH": torch.empty((T, F), dtype=torch.float32, device="cuda"),
        "dA": torch.empty((T, F), dtype=tdt, device="cuda"),
        "dX": torch.empty((T, D), dtype=torch.float32, device="cuda"),
    }
    host = {"W1t": W1t, "W2t": W2t, "dW1t": dW1t, "dW2t": dW2t}
    return tiling, ctx, p1, p2, bufs, host


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ffn_block_small(dtype):
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case ffn small", dtype)
    tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, dtype, seed=20, w_std=0.05)
    torch.cuda.synchronize()
    # forward, keeping a copy of A/H from the first forward to compare with the recompute
    ctx.fwd_gelu(p1, b["X"], b["A"], b["H"])
    ctx.sync()
    A0, H0 = b["A"].clone(), b["H"].clone()
    tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"],
                          b["dX"], b["Yr"])
    ctx.sync()
    assert torch.equal(A0, b["A"]) and torch.equal(H0, b["H"]), "recomputed A/H differ"
    assert torch.equal(b["Y"], b["Yr"]), "recomputed Y differs"
    r = oracle.ffn_fwd_bwd(host_bits(b["X"]), host_bits(h["W1t"]), host_bits(h["W2t"]),
                           host_bits(b["dY"]), dtype)
    tol = 2e-3 if dtype == "f16" else 8e-3
    for k in ("A", "H", "Y", "dA"):
        assert_close(values(b[k], dtype), r[k], k, tol)
    assert_close(values(b["dH"], dtype), r["dH"], "dH", 2e-3 if dtype == "f16" else 8e-3)
    assert_close(values(b["dX"], dtype), r["dX"], "dX", tol)
    assert_close(values(h["dW1t"], dtype), r["dW1t"], "dW1", tol)
    assert_close(values(h["dW2t"], dtype), r["dW2t"], "dW2", tol)
    ctx.close()


def test_gelu_bwd_kernel_elementwise():
    # dA = RNE(dH * GeLU'(A)) on a ragged count, against the oracle's GeLU'
    tiling = lib()
    count = 10007
    A = inputs.new((1, count), "f16", "gaussian", 21, "X", device="cuda").view(-1)
    A.mul_(3)
    dH = torch.randn(count, generator=torch.Generator(device="cuda").manual_seed(21), device="cuda")
    dA = torch.empty_like(A)
    Wt = tiling.host_tensor((8, 8), torch.float16)
    plan = tiling.Plan(1, 8, 8, 1, 1, "f16", Wt)
    ctx = tiling.Context(plan)
    torch.cuda.synchronize()
    ctx.gelu_bwd("f16", dH, A, dA, count)
    ctx.sync()
    a = oracle.decode(host_bits(A), "f16")
    ref = dH.cpu().numpy().astype(np.float64) * oracle.gelu_grad(a)
    got = oracle.decode(host_bits(dA), "f16")
    # fp32 evaluation then one fp16 rounding: within one fp16 ulp of the exact value
    ulp = np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10
    assert np.all(np.abs(got - ref) <= ulp), float(np.max(np.abs(got - ref) / ulp))
    ctx.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gelu_epilogue_every_16bit_input(dtype):
    # X = e_0 and column m of W holds the 16-bit value with bits m in row 0
    # (zeros elsewhere): A[0][m] is that value, so H is GeLU at every 16-bit
    # input, and must be the oracle's fp64 GeLU rounded once (a mismatch is
    # allowed only where the fp64 value sits within 1e-12 of a rounding tie,
    # where the last ulp of the two erfc implementations decides)
    T, K, M, N, d = 1, 8, 65536, 1, 1
    say("case gelu table", dtype)
    tiling = lib()
    tdt = inputs.torch_dtype(dtype)
    Wt = tiling.host_tensor((M, K), tdt)
    w = Wt.view(torch.int16)
    w.zero_()
    w[:, 0] = torch.arange(M, dtype=torch.int32).to(torch.int16)
    X = torch.zeros((T, K), dtype=tdt, device="cuda")
    X[0, 0] = 1
    plan = tiling.Plan(T, K, M, N, d, dtype, Wt)
    ctx = tiling.Context(plan)
    A = torch.empty((T, M), dtype=tdt, device="cuda")
    H = torch.empty_like(A)
    torch.cuda.synchronize()
    ctx.fwd_gelu(plan, X, A, H)
    ctx.sync()
    a_bits, h_bits = host_bits(A).ravel(), host_bits(H).ravel()
    w_val = oracle.decode(np.arange(M, dtype=np.uint16), dtype)
    a_val = oracle.decode(a_bits, dtype)
    fin = np.isfinite(w_val)
    assert np.array_equal(a_val[fin], w_val[fin]), "A is not the input value"
    fin = np.isfinite(a_val)
    h_ref = oracle.gelu(a_val[fin])
    want = oracle.encode(h_ref, dtype)
    got = h_bits[fin]
    bad = np.nonzero(got != want)[0]
    say("  %d finite inputs, %d differ from the oracle" % (fin.sum(), bad.size))
    if bad.size:
        g, o, r = oracle.decode(got[bad], dtype), oracle.decode(want[bad], dtype), h_ref[bad]
        assert np.all(np.abs(r - 0.5 * (g + o)) <= 1e-12 * np.abs(r)), "H off the oracle away from a tie"
        assert bad.size <= 4, bad.size
    inf_pos = np.nonzero(np.isposinf(a_val))[0]
    assert inf_pos.size and np.all(np.isposinf(oracle.decode(h_bits[inf_pos], dtype)))
    ctx.close()
    plan.close()
