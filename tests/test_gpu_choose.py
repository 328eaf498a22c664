"""The tile-width choice on the GPU: rates measured at a few widths, the
planner's pick from them (zi_plan_choose), and that pick run through the ring
bit-exact against the oracle (small integers: every sum exact)."""
import numpy as np
import pytest
import torch

import oracle
from zi_testlib import host_bits, lib, make_linear_inputs, say

pytestmark = pytest.mark.gpu


def measure(tiling, T, K, M, width, X, Wt, dY):
    """Per-launch rates of the three products and of the tile copies at one
    tile width (d = 2, no budget), from the context's timing events."""
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, M // width, 2, "f16", Wt, dWt)
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y)
    ctx.bwd(plan, X, dY, dX)
    ctx.sync()
    ctx.set_timing(True)
    ctx.reset_stats()
    for _ in range(2):
        ctx.fwd(plan, X, Y)
        ctx.bwd(plan, X, dY, dX)
    ctx.sync()
    st = ctx.stats()
    ctx.close()
    plan.close()
    k = st["kinds"]

    def rate(name):
        return k[name]["flops"] / (k[name]["ms"] * 1e-3)

    return (rate("gemm_fwd"), rate("gemm_dx"), rate("gemm_dw"),
            st["h2d_bytes"] / (st["h2d_ms"] * 1e-3), st["d2h_bytes"] / (st["d2h_ms"] * 1e-3))


def test_chosen_tiling_runs_bit_exact():
    from offload_memory_centric_amd import zi
    tiling = lib()
    T, K, M = 1024, 2048, 8192
    widths = [512, 1024, 2048, 4096]
    budget = 3 * K * 2048 * 2  # three tiles of the middle width
    say("case tile-width choice: measuring", widths)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=60)
    rows = [measure(tiling, T, K, M, w, X, Wt, dY) for w in widths]
    fwd, dx, dw, h2d, d2h = (list(c) for c in zip(*rows))
    say("  fwd TFLOP/s", [round(r / 1e12, 1) for r in fwd], "h2d GB/s", [round(r / 1e9, 1) for r in h2d])
    problem = zi.zi_problem(T=T, K=K, M=M, N=1, d=1, dtype=zi.DTYPE_CODES["f16"], flags=0,
                            device_budget_bytes=budget, W_host=None, dW_host=None)
    choice, table = zi.zi_plan_choose(problem, widths, fwd, dx, dw, float(np.median(h2d)), float(np.median(d2h)),
                                      1, 3, h2d=h2d, d2h=d2h)
    say("  chosen", choice)
    assert choice["n"] in widths and choice["N"] * choice["n"] == M
    assert choice["ring_bytes"] <= budget
    assert choice["t_step_s"] == min(c["t_step_s"] for c in table)

    # the chosen tiling, under the same budget, against the oracle
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, choice["N"], choice["d"], "f16", Wt, dWt, budget=budget)
    assert plan.info.ring_bytes == choice["ring_bytes"] and plan.info.dw_slots == choice["dw_slots"]
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y)
    ctx.bwd(plan, X, dY, dX)
    ctx.sync()
    Xb, Wb, dYb = host_bits(X), host_bits(Wt), host_bits(dY)
    Yr = oracle.linear_fwd(Xb, Wb, "f16")
    dXr, dWr = oracle.linear_bwd(Xb, Wb, dYb, "f16")
    assert np.array_equal(host_bits(Y), oracle.encode(Yr, "f16")), "Y"
    assert np.array_equal(dX.cpu().numpy().astype(np.float64), dXr), "dX"
    assert np.array_equal(host_bits(dWt), oracle.encode(dWr, "f16")), "dW"
    ctx.close()
    plan.close()
