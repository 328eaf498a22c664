"""The ring's ordering and its stall accounting under the context's debug
aids: released slots poisoned with NaNs before they are reused (a premature
reuse would show in the results), and a host-side delay before every tile
copy (the stall it causes must show in the accounting and match the model)."""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import host_bits, lib, make_linear_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,d,budget_tiles", [(4, 2, 0), (4, 1, 0), (8, 3, 0), (4, 2, 2), (5, 2, 0)])
def test_poisoned_slots_change_nothing(N, d, budget_tiles):
    # two forward + backward steps back to back (the ring carries over), with
    # separate gradient slots, the gradient in the weight slot (budget of two
    # tiles) and an odd tile count (a tile left out of the dX pairs)
    T, K, M = 128, 512, 2560 if N == 5 else 2048
    tiling = lib()
    say("case poison N", N, "d", d, "budget tiles", budget_tiles)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=11)
    dWt = tiling.host_tensor((M, K), torch.float16)
    budget = budget_tiles * K * (M // N) * 2
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, dWt, budget=budget)
    ctx = tiling.Context(plan)
    ctx.set_debug(poison=True)
    Ys = [torch.empty((T, M), dtype=torch.float16, device="cuda") for _ in range(2)]
    dXs = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for s in range(2):
        ctx.fwd(plan, X, Ys[s])
        ctx.bwd(plan, X, dY, dXs[s])
    ctx.sync()
    Xb, Wb, dYb = host_bits(X), host_bits(Wt), host_bits(dY)
    Y = oracle.encode(oracle.linear_fwd(Xb, Wb, "f16"), "f16")
    dX, dW = oracle.linear_bwd(Xb, Wb, dYb, "f16")
    for s in range(2):
        assert np.array_equal(host_bits(Ys[s]), Y), "Y of step %d" % (s + 1)
        assert np.array_equal(dXs[s].cpu().numpy().astype(np.float64), dX), "dX of step %d" % (s + 1)
    assert np.array_equal(host_bits(dWt), oracle.encode(dW, "f16")), "dW"
    ctx.close()
    plan.close()


def test_poisoned_ffn_block_equals_plain():
    from test_gpu_ffn import ffn_setup
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case poison ffn")
    tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, "f16", seed=42, w_std=0.05)
    keys = ("A", "H", "Y", "Yr", "dH", "dA", "dX")
    out = []
    for poison in (False, True):
        ctx.set_debug(poison=poison)
        torch.cuda.synchronize()
        for _ in range(2):
            tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"], b["dX"],
                                  b["Yr"])
        ctx.sync()
        out.append(({k: b[k].clone() for k in keys}, host_bits(h["dW1t"]).copy(), host_bits(h["dW2t"]).copy()))
        for k in keys:
            b[k].zero_()
    for k in keys:
        assert torch.equal(out[0][0][k], out[1][0][k]), k
    assert np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])
    ctx.close()


def test_copy_delay_shows_as_stall_and_matches_the_model():
    # every copy held 20 ms on the host: the products (microseconds here)
    # wait for every tile, so the pass is N copies long and the compute stream
    # idles nearly all of it; the ring's timing model, given a link that takes
    # 20 ms per tile, predicts the same pass time
    T, K, M, N, d = 128, 512, 2048, 4, 2
    delay = 20000
    tiling = lib()
    say("case copy delay")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=12)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, None)
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    ctx.fwd(plan, X, Y)
    ctx.sync()
    ctx.set_debug(copy_delay_us=delay)
    ctx.set_timing(True)
    ctx.reset_stats()
    ctx.fwd(plan, X, Y)
    ctx.sync()
    st = ctx.stats()
    ctx.set_timing(False)
    ctx.set_debug()
    Xb, Wb = host_bits(X), host_bits(Wt)
    assert np.array_equal(host_bits(Y), oracle.encode(oracle.linear_fwd(Xb, Wb, "f16"), "f16"))
    stall = 1.0 - st["compute_busy_ms"] / st["span_ms"]
    say("  span %.1f ms, busy %.3f ms, stall %.3f" % (st["span_ms"], st["compute_busy_ms"], stall))
    # the span runs from the first copy's start (after its delay) to the last product
    assert st["span_ms"] >= (N - 1) * delay / 1000.0
    assert stall > 0.95
    per_tile = plan.info.tile_bytes / (delay * 1e-6)
    pred = plan.predict(0, 1e15, per_tile)
    say("  predicted pass %.1f ms" % (pred.t_pass_s * 1e3))
    assert abs(pred.t_pass_s * 1e3 - (st["span_ms"] + delay / 1000.0)) < 0.25 * pred.t_pass_s * 1e3
    ctx.close()
    plan.close()


def test_timed_records_match_the_totals():
    # the per-launch records add up to zi_ctx_stats' totals, kernels in launch
    # order, copies after them, every interval inside the timed span
    T, K, M, N, d = 256, 512, 2048, 4, 2
    tiling = lib()
    say("case timed records")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=13)
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, dWt)
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ctx.set_timing(True)
    ctx.reset_stats()
    ctx.fwd(plan, X, Y)
    ctx.bwd(plan, X, dY, dX)
    st = ctx.stats()
    recs = ctx.timed_records()
    ctx.set_timing(False)
    kinds = list(st["kinds"])
    ker = [r for r in recs if r["what"] == "kernel"]
    assert len(ker) == sum(v["launches"] for v in st["kinds"].values())
    assert [r["what"] for r in recs] == ["kernel"] * len(ker) + [r["what"] for r in recs[len(ker):]]
    assert sum(1 for r in recs if r["what"] == "h2d") == st["h2d_copies"] == 2 * N
    assert sum(1 for r in recs if r["what"] == "d2h") == st["d2h_copies"] == N
    assert sum(r["rows"] for r in recs if r["what"] == "h2d") == st["h2d_bytes"]
    for name, v in st["kinds"].items():
        ms = sum(r["end_ms"] - r["start_ms"] for r in ker if kinds[r["kind"]] == name)
        assert ms == pytest.approx(v["ms"], rel=1e-6, abs=1e-6), name
    lo = min(r["start_ms"] for r in recs)
    hi = max(r["end_ms"] for r in recs)
    assert all(r["end_ms"] >= r["start_ms"] for r in recs)
    assert hi - lo == pytest.approx(st["span_ms"], rel=1e-6, abs=1e-6)
    assert [kinds[r["kind"]] for r in ker[:N]] == ["gemm_fwd"] * N
    ctx.close()
    plan.close()
