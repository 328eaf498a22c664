"""Forward passes on two product streams (zi_ctx_set_second_stream): the
results equal the oracle's on exact inputs and the one-stream results on the
feed-forward block, also with released slots poisoned (a product that read a
slot after its reuse began would see NaNs)."""
import numpy as np
import pytest
import torch

import oracle
from zi_testlib import host_bits, lib, make_linear_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,d", [(4, 2), (5, 2), (8, 3), (1, 1), (3, 1)])
@pytest.mark.parametrize("poison", [False, True])
def test_two_streams_bit_exact(N, d, poison):
    T, K = 128, 512
    M = 512 * N
    tiling = lib()
    say("case overlap N", N, "d", d, "poison", poison)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=13)
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, dWt)
    ctx = tiling.Context(plan, overlap=True)
    ctx.set_debug(poison=poison)
    Ys = [torch.empty((T, M), dtype=torch.float16, device="cuda") for _ in range(3)]
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Ys[0])
    ctx.fwd(plan, X, Ys[1])     # two forward passes back to back
    ctx.bwd(plan, X, dY, dX)
    ctx.fwd(plan, X, Ys[2])
    ctx.sync()
    Xb, Wb, dYb = host_bits(X), host_bits(Wt), host_bits(dY)
    Y = oracle.encode(oracle.linear_fwd(Xb, Wb, "f16"), "f16")
    dXr, dW = oracle.linear_bwd(Xb, Wb, dYb, "f16")
    for k in range(3):
        assert np.array_equal(host_bits(Ys[k]), Y), "Y of pass %d" % k
    assert np.array_equal(dX.cpu().numpy().astype(np.float64), dXr)
    assert np.array_equal(host_bits(dWt), oracle.encode(dW, "f16"))
    ctx.close()
    plan.close()


def test_ffn_block_two_streams_equals_one():
    from test_gpu_ffn import ffn_setup
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case overlap ffn")
    keys = ("A", "H", "Y", "Yr", "dH", "dA", "dX")
    out = []
    for overlap in (False, True):
        tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, "f16", seed=43, w_std=0.05)
        ctx.close()
        big = p1 if p1.info.ring_bytes >= p2.info.ring_bytes else p2
        ctx = tiling.Context(big, overlap=overlap)
        torch.cuda.synchronize()
        for _ in range(2):
            tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"], b["dX"],
                                  b["Yr"])
        ctx.sync()
        out.append(({k: b[k].clone() for k in keys}, host_bits(h["dW1t"]).copy(), host_bits(h["dW2t"]).copy()))
        ctx.close()
    for k in keys:
        assert torch.equal(out[0][0][k], out[1][0][k]), k
    assert np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])
