"""GPU parity of the feed-forward block (up-projection, GeLU, down-projection)
with activation checkpointing, against the oracle's chain (small shapes)."""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import TOL, assert_close, host_bits, lib, make_linear_inputs, say, stored_tol, values

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


def run_block_f32(tiling, T, D, F, N1, N2, d, dtype, b, h):
    """The same block step with every result left in fp32 where the method
    rounds it: A from the fused forward, Y and Yr, dW1 and dW2 (plans with
    f32_out), dA from the GeLU backward.  The 16-bit A of the first run feeds
    the GeLU backward, as in the method; the rest is recomputed."""
    tdt = inputs.torch_dtype(dtype)
    dW1f = tiling.host_tensor((F, D), torch.float32)
    dW2f = tiling.host_tensor((D, F), torch.float32)
    q1 = tiling.Plan(T, D, F, N1, d, dtype, h["W1t"], dW1f, f32_out=True)
    q2 = tiling.Plan(T, F, D, N2, d, dtype, h["W2t"], dW2f, f32_out=True)
    ctx = tiling.Context(q1 if q1.info.ring_bytes >= q2.info.ring_bytes else q2)
    f = {
        "A": torch.empty((T, F), dtype=torch.float32, device="cuda"),
        "H": torch.empty((T, F), dtype=tdt, device="cuda"),
        "Y": torch.empty((T, D), dtype=torch.float32, device="cuda"),
        "Yr": torch.empty((T, D), dtype=torch.float32, device="cuda"),
        "dH": torch.empty((T, F), dtype=torch.float32, device="cuda"),
        "dA": torch.empty((T, F), dtype=torch.float32, device="cuda"),
        "dA16": torch.empty((T, F), dtype=tdt, device="cuda"),
        "dX": torch.empty((T, D), dtype=torch.float32, device="cuda"),
    }
    torch.cuda.synchronize()
    ctx.fwd_gelu(q1, b["X"], f["A"], f["H"])
    ctx.fwd(q2, f["H"], f["Y"])
    ctx.bwd_recompute(q2, f["H"], b["dY"], f["dH"], f["Yr"])
    ctx.gelu_bwd(dtype, f["dH"], b["A"], f["dA"], T * F)
    ctx.gelu_bwd(dtype, f["dH"], b["A"], f["dA16"], T * F)
    ctx.bwd(q1, b["X"], f["dA16"], f["dX"])
    ctx.sync()
    f["dW1t"], f["dW2t"] = dW1f, dW2f
    ctx.close()
    q1.close()
    q2.close()
    return f


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
    # results the method keeps in fp32, for both formats
    assert_close(values(b["dH"], dtype), r["dH"], "dH")
    assert_close(values(b["dX"], dtype), r["dX"], "dX")
    # the stored 16-bit results, raw (bf16: bounded as stored_tol derives)
    for k, u in (("A", 1.0), ("H", 2.13), ("Y", 0.5), ("dA", 2.13)):
        assert_close(values(b[k], dtype), r[k], k, stored_tol(r[k], dtype, u))
    assert_close(values(h["dW1t"], dtype), r["dW1t"], "dW1", stored_tol(r["dW1t"], dtype, 0.5))
    assert_close(values(h["dW2t"], dtype), r["dW2t"], "dW2", stored_tol(r["dW2t"], dtype, 0.5))

    # The fp32 epilogues at the 2e-3 bar, and every stored 16-bit result one
    # RNE rounding of its fp32 form (bit-exact).
    f = run_block_f32(tiling, T, D, F, N1, N2, d, dtype, b, h)
    tdt = inputs.torch_dtype(dtype)
    assert torch.equal(f["H"], b["H"]) and torch.equal(f["dH"], b["dH"])
    assert torch.equal(f["dA16"], b["dA"]) and torch.equal(f["dX"], b["dX"])
    assert torch.equal(f["Y"], f["Yr"]), "recomputed fp32 Y differs"
    assert torch.equal(f["A"].to(tdt), b["A"]), "A is not RNE of its fp32 accumulator"
    assert torch.equal(f["Y"].to(tdt), b["Y"]), "Y is not RNE of its fp32 accumulator"
    assert torch.equal(f["dA"].to(tdt), b["dA"]), "dA is not RNE of its fp32 product"
    assert torch.equal(f["dW1t"].to(tdt), h["dW1t"]), "dW1 is not RNE of its fp32 accumulator"
    assert torch.equal(f["dW2t"].to(tdt), h["dW2t"]), "dW2 is not RNE of its fp32 accumulator"
    assert_close(values(f["A"], dtype), r["A_exact"], "A fp32")
    assert_close(values(f["Y"], dtype), r["Y"], "Y fp32")
    assert_close(values(f["dW1t"], dtype), r["dW1t"], "dW1 fp32")
    assert_close(values(f["dW2t"], dtype), r["dW2t"], "dW2 fp32")
    # A's rounding is unique except where the exact product lies within the
    # fp32 sum's error of a rounding boundary; there the two sides may hold
    # different values (several units apart where the sum nearly cancels and
    # its fp32 error exceeds the 16-bit spacing of the tiny result).  Where
    # they agree, H is unique (bit-exact) and dA's fp32 product meets the bar;
    # where they do not, the fp32 A lies within the bound of any fp32 sum of K
    # products, K 2^-24 sum_k |x_k w_k|, of the exact one, and dA within
    # |dH| max|GeLU''| |dA_in| of the oracle's (0.8 = GeLU''(0)).
    a_gpu = host_bits(b["A"]).astype(np.int64)
    a_ref = oracle.encode(r["A"], dtype).astype(np.int64)
    same = a_gpu == a_ref
    nd = int((~same).sum())
    say("  A: %d of %d elements round to another 16-bit value than the oracle's" % (nd, same.size))
    assert nd <= max(4, same.size // 1000), nd
    if nd:
        absx = np.abs(oracle.decode(host_bits(b["X"]), dtype))
        absw = np.abs(oracle.decode(host_bits(h["W1t"]), dtype))
        bound = D * 2.0 ** -24 * (absx @ absw.T)
        a32 = values(f["A"], dtype)
        assert np.all(np.abs(a32 - r["A_exact"])[~same] <= bound[~same]), "fp32 A beyond the sum's error"
    h_gpu = host_bits(b["H"])
    assert np.array_equal(h_gpu[same], oracle.encode(r["H"], dtype)[same]), "H differs where A agrees"
    dA32 = values(f["dA"], dtype)
    assert_close(dA32[same], r["dA_exact"][same], "dA fp32")
    if nd:
        dA_in = np.abs(values(b["A"], dtype) - r["A"])[~same]
        bound = np.abs(r["dH"][~same]) * 0.8 * dA_in + TOL * np.abs(r["dA_exact"]).max()
        assert np.all(np.abs(dA32[~same] - r["dA_exact"][~same]) <= bound)
    ctx.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gelu_bwd_kernel_elementwise(dtype):
    # dA = RNE(dH * GeLU'(A)) on a ragged count, against the oracle's GeLU';
    # the fp32 form is the product before that rounding
    tiling = lib()
    count = 10007
    tdt = inputs.torch_dtype(dtype)
    A = inputs.new((1, count), dtype, "gaussian", 21, "X", device="cuda").view(-1)
    A.mul_(3)
    dH = torch.randn(count, generator=torch.Generator(device="cuda").manual_seed(21), device="cuda")
    dA = torch.empty_like(A)
    dA32 = torch.empty(count, dtype=torch.float32, device="cuda")
    Wt = tiling.host_tensor((8, 8), tdt)
    plan = tiling.Plan(1, 8, 8, 1, 1, dtype, Wt)
    ctx = tiling.Context(plan)
    torch.cuda.synchronize()
    ctx.gelu_bwd(dtype, dH, A, dA, count)
    ctx.gelu_bwd(dtype, dH, A, dA32, count)
    ctx.sync()
    a = oracle.decode(host_bits(A), dtype)
    ref = dH.cpu().numpy().astype(np.float64) * oracle.gelu_grad(a)
    got = oracle.decode(host_bits(dA), dtype)
    # fp32 evaluation then one rounding: within one ulp of the exact value
    mant, tiny = (10, 2.0 ** -14) if dtype == "f16" else (7, 2.0 ** -126)
    u = np.maximum(np.abs(ref), tiny) * 2.0 ** -mant
    assert np.all(np.abs(got - ref) <= u), float(np.max(np.abs(got - ref) / u))
    # the fp32 product: Phi(a) and a phi(a) each carry a few fp32 roundings,
    # amplified by at most 1 + a^2 (the condition of erfc and exp here), so the
    # error is bounded by |dH| (Phi + |a| phi) (1 + a^2) 2^-20 plus the product's
    # own rounding; where GeLU' nearly cancels (a near -0.75) this absolute
    # part is what holds
    g32 = dA32.cpu().numpy().astype(np.float64)
    dh = np.abs(dH.cpu().numpy().astype(np.float64))
    parts = oracle.gelu(a) / np.where(a == 0, 1.0, a)  # Phi(a)
    parts = np.where(a == 0, 0.5, parts) + np.abs(a) * np.exp(-0.5 * a * a) / np.sqrt(2 * np.pi)
    assert np.all(np.abs(g32 - ref) <= dh * parts * (1 + a * a) * 2.0 ** -20 + np.abs(ref) * 2.0 ** -22)
    assert torch.equal(dA32.to(tdt), dA), "dA is not RNE of its fp32 product"
    ctx.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gelu_bwd_every_16bit_input(dtype):
    # A takes every finite 16-bit value (GeLU' looked up: from LDS for
    # |A| < 16, from the global table beyond), dH a random value each; the same
    # bounds as the elementwise test, against the oracle's fp64 GeLU'.  Below
    # a = -13.3 GeLU'(a) lies under fp32's smallest normal value 2^-126, where
    # fp32 carries only absolute accuracy (the terms of Phi(a) + a phi(a)
    # are subnormal, and exp may return 0): there an fp32 evaluation is off by
    # up to 2^-126 |dH|, and the product's own rounding by up to 2^-150
    tiling = lib()
    tdt = inputs.torch_dtype(dtype)
    codes = np.arange(65536, dtype=np.uint16)
    a_all = oracle.decode(codes, dtype)
    keep = np.isfinite(a_all)
    codes, a = codes[keep], a_all[keep]
    count = len(codes)
    A = torch.from_numpy(codes.view(np.int16).copy()).view(tdt).cuda()
    dH = torch.randn(count, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
    dA = torch.empty_like(A)
    dA32 = torch.empty(count, dtype=torch.float32, device="cuda")
    plan = tiling.Plan(1, 8, 8, 1, 1, dtype, tiling.host_tensor((8, 8), tdt))
    ctx = tiling.Context(plan)
    torch.cuda.synchronize()
    ctx.gelu_bwd(dtype, dH, A, dA, count)
    ctx.gelu_bwd(dtype, dH, A, dA32, count)
    ctx.sync()
    ref = dH.cpu().numpy().astype(np.float64) * oracle.gelu_grad(a)
    g32 = dA32.cpu().numpy().astype(np.float64)
    dh = np.abs(dH.cpu().numpy().astype(np.float64))
    phi = oracle.gelu(a) / np.where(a == 0, 1.0, a)
    parts = np.where(a == 0, 0.5, phi) + np.abs(a) * np.exp(-0.5 * a * a) / np.sqrt(2 * np.pi)
    bound = dh * parts * (1 + a * a) * 2.0 ** -20 + np.abs(ref) * 2.0 ** -22
    bound = bound + np.where(np.abs(oracle.gelu_grad(a)) < 2.0 ** -126, dh * 2.0 ** -126 + 2.0 ** -149, 0.0)
    bad = np.flatnonzero(np.abs(g32 - ref) > bound)
    assert len(bad) == 0, "%d over the bound, e.g. %s" % (len(bad), [
        (float(a[i]), float(g32[i]), float(ref[i]), float(bound[i])) for i in bad[:12]])
    assert torch.equal(dA32.to(tdt), dA), "dA is not RNE of its fp32 product"
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


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,M,N", [(4096, 512, 1024, 1), (8192, 512, 4608, 2)])
def test_split_gelu_forward_bit_exact(dtype, T, K, M, N):
    # The GeLU forward with the split workspace: 16 x 4 = 64 tiles, all taken
    # as two half-reductions (K = 256 each), and 32 x 9 = 288 tiles per weight
    # tile, one full round of 256 and 32 split.  Small integers make every sum
    # exact, so A and H equal the unsplit launch's bit for bit and A is the
    # oracle's product rounded once; two calls in a row check that each
    # launch leaves its arrival counters cleared for the next.  With two
    # weight tiles and the second product stream the tiles alternate between
    # the two streams' split workspaces.
    say("case split GeLU forward", dtype, T, K, M, N)
    tiling = lib()
    tdt = inputs.torch_dtype(dtype)
    X, Wt, _ = make_linear_inputs(T, K, M, dtype, "small_int", seed=41)
    outs = []
    for split, overlap in ((True, False), (False, False), (True, True)):
        plan = tiling.Plan(T, K, M, N, 2, dtype, Wt)
        ctx = tiling.Context(plan, gelu_split=split, overlap=overlap)
        got = []
        for _ in range(2):
            A = torch.empty((T, M), dtype=tdt, device="cuda")
            H = torch.empty_like(A)
            torch.cuda.synchronize()
            ctx.fwd_gelu(plan, X, A, H)
            ctx.sync()
            got.append((host_bits(A), host_bits(H)))
        outs.append(got)
        ctx.close()
        plan.close()
    (a0, h0), (a1, h1) = outs[0]
    assert np.array_equal(a0, a1) and np.array_equal(h0, h1), "second split launch differs from the first"
    assert np.array_equal(a0, outs[1][0][0]), "split A differs from the unsplit launch"
    assert np.array_equal(h0, outs[1][0][1]), "split H differs from the unsplit launch"
    for k in range(2):
        assert np.array_equal(a0, outs[2][k][0]) and np.array_equal(h0, outs[2][k][1]), "two product streams"
    ref = oracle.linear_fwd(host_bits(X), host_bits(Wt), dtype)
    assert np.array_equal(a0, oracle.encode(ref, dtype)), "A against the oracle"
