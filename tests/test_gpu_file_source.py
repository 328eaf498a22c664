"""The tiled path with its weights read from files (the NVMe tier), on the
GPU: results bit-identical to the oracle's on exact inputs; on Gaussian ones
bit-identical to the same passes fed from pinned host memory and within the
2e-3 bar of the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import assert_close, host_bits, lib, make_linear_inputs, say, values

pytestmark = pytest.mark.gpu


def weight_file(tmp_path, name, W_host):
    tiling = lib()
    path = str(tmp_path / name)
    tiling.write_weight_file(path, W_host)
    return path


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,d,staging", [(4, 2, 2), (4, 1, 3), (8, 3, 4), (1, 1, 2)])
def test_linear_from_file_bit_exact(tmp_path, dtype, N, d, staging):
    # small integers: every sum exact, every stored result unique; three
    # forward + backward steps back to back, so the read-ahead crosses passes
    T, K, M, S = 128, 512, 2048, 3
    tiling = lib()
    say("case file source", dtype, "N", N, "d", d, "staging", staging)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=7)
    path = weight_file(tmp_path, "w.bin", Wt)
    W_bits = host_bits(Wt).copy()
    dWt = tiling.host_tensor((M, K), inputs.torch_dtype(dtype))
    plan = tiling.Plan(T, K, M, N, d, dtype, None, dWt)
    ctx = tiling.Context(plan)
    src = tiling.FileSource(plan, path, staging=staging, threads=3)
    ctx.attach_source(plan, src)
    Ys = [torch.empty((T, M), dtype=inputs.torch_dtype(dtype), device="cuda") for _ in range(S)]
    dXs = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(S)]
    torch.cuda.synchronize()
    for s in range(S):
        ctx.fwd(plan, X, Ys[s])
        ctx.bwd(plan, X, dY, dXs[s])
    ctx.sync()
    Xb, dYb = host_bits(X), host_bits(dY)
    Y = oracle.encode(oracle.linear_fwd(Xb, W_bits, dtype), dtype)
    dX, dW = oracle.linear_bwd(Xb, W_bits, dYb, dtype)
    for s in range(S):
        assert np.array_equal(host_bits(Ys[s]), Y), "Y of step %d" % (s + 1)
        assert np.array_equal(dXs[s].cpu().numpy().astype(np.float64), dX), "dX of step %d" % (s + 1)
    assert np.array_equal(host_bits(dWt), oracle.encode(dW, dtype)), "dW"
    st = src.stats()
    say("  source", st)
    assert st["restarts"] == 0
    # every tile is read at least once, and no request more than once (the
    # read-ahead may run a few tiles past the last pass); with a buffer per
    # tile exactly once: the buffers then hold the whole weight
    if staging >= N:
        assert st["tiles_read"] == N
    else:
        assert N <= st["tiles_read"] <= 2 * S * N + staging
    ctx.attach_source(plan, None)
    ctx.close()
    src.close()
    plan.close()


def test_ffn_block_from_files_equals_host(tmp_path):
    # the block with both weights read from files gives the same bits as the
    # block fed from pinned host memory (same kernels, same inputs)
    from test_gpu_ffn import ffn_setup
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case ffn from files")
    tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, "f16", seed=40, w_std=0.05)
    torch.cuda.synchronize()
    tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"], b["dX"], b["Yr"])
    ctx.sync()
    ref = {k: b[k].clone() for k in ("A", "H", "Y", "dH", "dA", "dX")}
    ref_dw = (host_bits(h["dW1t"]).copy(), host_bits(h["dW2t"]).copy())
    s1 = tiling.FileSource(p1, weight_file(tmp_path, "w1.bin", h["W1t"]), staging=3, threads=2)
    s2 = tiling.FileSource(p2, weight_file(tmp_path, "w2.bin", h["W2t"]), staging=2, threads=2)
    ctx.attach_source(p1, s1)
    ctx.attach_source(p2, s2)
    h["W1t"].zero_()  # the passes must not read the host copies any more
    h["W2t"].zero_()
    for k in ref:
        b[k].zero_()
    torch.cuda.synchronize()
    for _ in range(2):
        tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"], b["dX"],
                              b["Yr"])
    ctx.sync()
    for k in ref:
        assert torch.equal(b[k], ref[k]), k
    assert np.array_equal(host_bits(h["dW1t"]), ref_dw[0]) and np.array_equal(host_bits(h["dW2t"]), ref_dw[1])
    say("  sources", s1.stats(), s2.stats())
    for s in (s1, s2):
        assert s.stats()["restarts"] == 0
    ctx.attach_source(p1, None)
    ctx.attach_source(p2, None)
    ctx.close()
    s1.close()
    s2.close()


def test_source_and_optimizer_exclude_each_other(tmp_path):
    T, K, M = 128, 512, 2048
    tiling = lib()
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=8)
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, 4, 2, "f16", Wt, dWt)
    ctx = tiling.Context(plan)
    src = tiling.FileSource(plan, weight_file(tmp_path, "w.bin", Wt))
    adam = tiling.Adam(plan, threads=2)
    ctx.attach_source(plan, src)
    from offload_memory_centric_amd import zi
    with pytest.raises(zi.ZiError) as e:
        ctx.attach_adam(plan, adam)
    assert e.value.status == zi.ZI_ERR_STATE
    ctx.attach_source(plan, None)
    ctx.attach_adam(plan, adam)
    with pytest.raises(zi.ZiError) as e:
        ctx.attach_source(plan, src)
    assert e.value.status == zi.ZI_ERR_STATE
    ctx.attach_adam(plan, None)
    ctx.close()
    adam.close()
    src.close()
    plan.close()


def run_block(tiling, ctx, p1, p2, b, forward_only=False, w2_first=False):
    if w2_first:  # the down-projection's forward alone (an order the trace does not know)
        ctx.fwd(p2, b["H"], b["Y"])
        return
    if forward_only:
        ctx.fwd_gelu(p1, b["X"], b["A"], b["H"])
        ctx.fwd(p2, b["H"], b["Y"])
        return
    tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"], b["dX"], b["Yr"])


def test_ffn_block_through_one_tier(tmp_path):
    # both weights under one tier: the first step is recorded and read on
    # demand, the next ones read ahead along the trace; steps in another order
    # restart the read-ahead.  Every step gives the host-fed block's bits.
    from test_gpu_ffn import ffn_setup
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case ffn through a tier")
    tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, "f16", seed=41, w_std=0.05)
    torch.cuda.synchronize()
    run_block(tiling, ctx, p1, p2, b)
    ctx.sync()
    keys = ("A", "H", "Y", "dH", "dA", "dX")
    ref = {k: b[k].clone() for k in keys}
    ref_dw = (host_bits(h["dW1t"]).copy(), host_bits(h["dW2t"]).copy())
    # the oracle's block on the same weights, for the tier-fed steps below
    r = oracle.ffn_fwd_bwd(host_bits(b["X"]), host_bits(h["W1t"]).copy(), host_bits(h["W2t"]).copy(),
                           host_bits(b["dY"]), "f16")
    tier = tiling.Tier(staging=3, threads=2)
    s1 = tiling.FileSource(p1, weight_file(tmp_path, "w1.bin", h["W1t"]))
    s2 = tiling.FileSource(p2, weight_file(tmp_path, "w2.bin", h["W2t"]))
    tier.add(s1)
    tier.add(s2)
    ctx.attach_source(p1, s1)
    ctx.attach_source(p2, s2)
    h["W1t"].zero_()
    h["W2t"].zero_()

    def check(what, with_oracle=False):
        ctx.sync()
        if with_oracle:  # the tier-fed outputs themselves against the oracle
            for k in keys:
                assert_close(values(b[k], "f16"), r[k], "%s %s" % (what, k))
            assert_close(values(h["dW1t"], "f16"), r["dW1t"], what + " dW1")
            assert_close(values(h["dW2t"], "f16"), r["dW2t"], what + " dW2")
        for k in keys:
            assert torch.equal(b[k], ref[k]), (what, k)
            b[k].zero_()
        assert np.array_equal(host_bits(h["dW1t"]), ref_dw[0]), what
        assert np.array_equal(host_bits(h["dW2t"]), ref_dw[1]), what

    per_step = 3 * N1 + 2 * N2
    run_block(tiling, ctx, p1, p2, b)        # recorded, read on demand
    tier.step()
    check("recorded step", with_oracle=True)
    st = tier.stats()
    say("  after the recorded step", st)
    # the recorded step is served on demand, or from a buffer that still holds the tile
    assert st["trace_len"] == per_step and 0 < st["demand_reads"] <= per_step
    assert st["restarts"] == 0
    recorded_demand = st["demand_reads"]
    # the recorded order, as (source index << 32 | tile): W1 forward, W2
    # forward, W1 recomputed, W2 backward, W1 backward, each tile ascending
    from offload_memory_centric_amd import zi
    order = [(0, t) for t in range(N1)] + [(1, t) for t in range(N2)] + [(0, t) for t in range(N1)] + \
        [(1, t) for t in range(N2)] + [(0, t) for t in range(N1)]
    assert zi.zi_tier_trace_get(tier.handle) == [(s << 32) | t for s, t in order]
    for n in range(2):                       # replayed
        run_block(tiling, ctx, p1, p2, b)
        tier.step()
        check("replayed step %d" % n, with_oracle=(n == 1))
    st = tier.stats()
    say("  after two replayed steps", st)
    assert st["demand_reads"] == recorded_demand and st["restarts"] == 0
    assert st["tiles_read"] + st["hits"] >= 3 * per_step
    # a forward-only step ends inside the trace: the next step starts over
    run_block(tiling, ctx, p1, p2, b, forward_only=True)
    tier.step()
    ctx.sync()
    assert torch.equal(b["Y"], ref["Y"])
    run_block(tiling, ctx, p1, p2, b)
    tier.step()
    check("step after a forward-only one")
    # a request out of the trace's order restarts the read-ahead where it is
    run_block(tiling, ctx, p1, p2, b, w2_first=True)
    run_block(tiling, ctx, p1, p2, b)
    tier.step()
    check("step after an unpredicted pass", with_oracle=True)
    st = tier.stats()
    say("  at the end", st)
    assert st["restarts"] >= 2
    ctx.attach_source(p1, None)
    ctx.attach_source(p2, None)
    ctx.close()
    tier.close()
    s1.close()
    s2.close()


def test_read_error_fails_the_pass_and_sticks(tmp_path):
    # the file loses its second half after the source was made: the pass that
    # needs tile 2 reports ZI_ERR_IO, the context keeps the error, and closing
    # it waits for the work already enqueued
    T, K, M, N = 128, 512, 2048, 4
    tiling = lib()
    from offload_memory_centric_amd import zi
    say("case file read error")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=9)
    path = weight_file(tmp_path, "w.bin", Wt)
    plan = tiling.Plan(T, K, M, N, 2, "f16", None, None)
    ctx = tiling.Context(plan)
    src = tiling.FileSource(plan, path, staging=2, threads=2)
    os.truncate(path, 2 * plan.info.tile_bytes)
    ctx.attach_source(plan, src)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    with pytest.raises(zi.ZiError) as e:
        ctx.fwd(plan, X, Y)
    assert e.value.status == zi.ZI_ERR_IO
    with pytest.raises(zi.ZiError) as e:
        ctx.sync()
    assert e.value.status == zi.ZI_ERR_IO
    ctx.attach_source(plan, None)
    ctx.close()
    src.close()
    plan.close()
