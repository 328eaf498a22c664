"""The host Adam attached to a context, on the GPU: every tile's update starts
once its gradient has landed in host memory, and the next pass over the same
weight copies each tile only after its update has rewritten it.

The steps are enqueued back to back with no host synchronisation between
them, so a pass that copied a tile before its update finished would compute
with stale weights; the expected values of every step come from the oracle's
chain (forward and backward with that step's weights, then its Adam step).
"""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import assert_close, host_bits, lib, make_linear_inputs, say, stored_tol, values

pytestmark = pytest.mark.gpu

# the library takes its hyperparameters in fp32: the oracle gets the same values
HP32 = {k: float(np.float32(x)) for k, x in dict(lr=0.25, beta1=0.9, beta2=0.999, eps=1e-8).items()}


def stored(x, dtype, f32):
    """What a pass stores for exact values x: fp32, or one RNE into 16 bits."""
    return np.float32(x) if f32 else oracle.encode(x, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,d,f32_out", [(4, 2, False), (4, 1, False), (8, 3, False), (4, 2, True)])
def test_steps_back_to_back_bit_exact(dtype, N, d, f32_out):
    # X, W, dY with values in {-3..3} and lr = 1/4.  The gradient X^T dY does
    # not depend on W, so it is the same integer matrix every step, and with a
    # constant gradient each Adam step moves a weight by lr * sign(g) (bias
    # corrected moments give m_hat / sqrt(v_hat) = sign(g)).  The weights stay
    # multiples of 1/4 below 4 in magnitude, so every product and sum of every
    # step is exact in fp32 and each stored result is unique: all outputs of
    # all steps are compared bit for bit.
    T, K, M, S = 128, 512, 2048, 3
    tiling = lib()
    say("case adam back-to-back", dtype, "N", N, "d", d, "f32_out", f32_out)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=5)
    W0 = host_bits(Wt).copy()
    elem = torch.float32 if f32_out else inputs.torch_dtype(dtype)
    dWt = tiling.host_tensor((M, K), elem)
    plan = tiling.Plan(T, K, M, N, d, dtype, Wt, dWt, f32_out=f32_out)
    ctx = tiling.Context(plan)
    adam = tiling.Adam(plan, threads=4, **HP32)
    ctx.attach_adam(plan, adam)
    Ys = [torch.empty((T, M), dtype=elem, device="cuda") for _ in range(S)]
    dXs = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(S)]
    torch.cuda.synchronize()
    for s in range(S):
        ctx.fwd(plan, X, Ys[s])
        ctx.bwd(plan, X, dY, dXs[s])
    ctx.sync()  # also waits for the attached optimizer

    Xb, dYb = host_bits(X), host_bits(dY)
    _, g = oracle.linear_bwd(Xb, W0, dYb, dtype)
    g_stored = stored(g, dtype, f32_out)
    if f32_out:
        assert np.array_equal(dWt.numpy(), g_stored), "dW"
        g_used = g_stored.astype(np.float64)
    else:
        assert np.array_equal(host_bits(dWt), g_stored), "dW bits"
        g_used = oracle.decode(g_stored, dtype)
    om, omm, ov = oracle.decode(W0, dtype), np.zeros((M, K)), np.zeros((M, K))
    Wbits = W0
    for s in range(S):
        Y = oracle.linear_fwd(Xb, Wbits, dtype)
        dX, _ = oracle.linear_bwd(Xb, Wbits, dYb, dtype)
        got_Y = Ys[s].cpu().numpy() if f32_out else host_bits(Ys[s])
        assert np.array_equal(got_Y, stored(Y, dtype, f32_out)), "Y of step %d" % (s + 1)
        assert np.array_equal(dXs[s].cpu().numpy().astype(np.float64), dX), "dX of step %d" % (s + 1)
        om, omm, ov = oracle.adam_step(om, omm, ov, g_used, s + 1, **HP32)
        Wbits = oracle.encode(om, dtype)
        # the constant-gradient closed form of the oracle's chain
        want = oracle.encode(oracle.decode(W0, dtype) - HP32["lr"] * (s + 1) * np.sign(g_used), dtype)
        assert np.array_equal(Wbits, want), "oracle chain off the closed form at step %d" % (s + 1)
    master, m, v = adam.master.numpy(), adam.m.numpy(), adam.v.numpy()
    assert np.max(np.abs(master - om)) <= 2e-6, np.max(np.abs(master - om))
    assert np.max(np.abs(m - omm)) <= 1e-6 * np.max(np.abs(omm))
    assert np.max(np.abs(v - ov)) <= 1e-6 * np.max(np.abs(ov))
    assert np.array_equal(host_bits(Wt), Wbits), "W after the last step"
    assert np.array_equal(host_bits(Wt), oracle.encode(master.astype(np.float64), dtype))
    st = adam.stats()
    assert st["tiles_done"] == S * N, st
    ctx.close()
    adam.close()
    plan.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ffn_block_then_forward_sees_the_update(dtype):
    # One step of the feed-forward block with an optimizer on each weight,
    # then the next forward pass, all enqueued without a host synchronisation:
    # the gradients and the updates follow the oracle, and the second forward
    # computes with the updated weights, far from what the old ones give.
    from test_gpu_ffn import ffn_setup
    T, D, F, N1, N2, d = 96, 256, 1024, 4, 4, 2
    say("case adam ffn", dtype)
    tiling, ctx, p1, p2, b, h = ffn_setup(T, D, F, N1, N2, d, dtype, seed=30, w_std=0.05)
    hp = dict(HP32, lr=float(np.float32(1e-2)))
    W1_0, W2_0 = host_bits(h["W1t"]).copy(), host_bits(h["W2t"]).copy()
    a1 = tiling.Adam(p1, threads=4, **hp)
    a2 = tiling.Adam(p2, threads=4, **hp)
    ctx.attach_adam(p1, a1)
    ctx.attach_adam(p2, a2)
    tdt = inputs.torch_dtype(dtype)
    A2 = torch.empty((T, F), dtype=tdt, device="cuda")
    H2 = torch.empty((T, F), dtype=tdt, device="cuda")
    Y2 = torch.empty((T, D), dtype=tdt, device="cuda")
    torch.cuda.synchronize()
    tiling.ffn_block_step(ctx, p1, p2, b["X"], b["A"], b["H"], b["Y"], b["dY"], b["dH"], b["dA"],
                          b["dX"], b["Yr"])
    ctx.fwd_gelu(p1, b["X"], A2, H2)
    ctx.fwd(p2, H2, Y2)
    ctx.sync()

    Xb, dYb = host_bits(b["X"]), host_bits(b["dY"])
    r0 = oracle.ffn_fwd_bwd(Xb, W1_0, W2_0, dYb, dtype)
    assert_close(values(h["dW1t"], dtype), r0["dW1t"], "dW1", stored_tol(r0["dW1t"], dtype, 0.5))
    assert_close(values(h["dW2t"], dtype), r0["dW2t"], "dW2", stored_tol(r0["dW2t"], dtype, 0.5))
    for a, W0, g in ((a1, W1_0, h["dW1t"]), (a2, W2_0, h["dW2t"])):
        # the update of the gradient the library stored, against the oracle's Adam
        om, omm, ov = oracle.adam_step(oracle.decode(W0, dtype), 0.0, 0.0, values(g, dtype), 1, **hp)
        master = a.master.numpy()
        assert np.max(np.abs(master - om)) <= 1e-7, np.max(np.abs(master - om))
        assert np.max(np.abs(a.m.numpy() - omm)) <= 1e-6 * np.max(np.abs(omm))
        assert np.max(np.abs(a.v.numpy() - ov)) <= 1e-6 * np.max(np.abs(ov))
    assert np.array_equal(host_bits(h["W1t"]), oracle.encode(a1.master.numpy().astype(np.float64), dtype))
    assert np.array_equal(host_bits(h["W2t"]), oracle.encode(a2.master.numpy().astype(np.float64), dtype))
    r1 = oracle.ffn_fwd_bwd(Xb, host_bits(h["W1t"]), host_bits(h["W2t"]), dYb, dtype)
    assert_close(values(A2, dtype), r1["A"], "A step 2", stored_tol(r1["A"], dtype, 1.0))
    assert_close(values(H2, dtype), r1["H"], "H step 2", stored_tol(r1["H"], dtype, 2.13))
    tol = stored_tol(r1["Y"], dtype, 0.5)
    assert_close(values(Y2, dtype), r1["Y"], "Y step 2", tol)
    stale = np.abs(values(Y2, dtype) - r0["Y"]).max()
    assert stale > 5 * tol * np.abs(r1["Y"]).max(), "the second forward looks like the old weights"
    ctx.close()
    for x in (a1, a2, p1, p2):
        x.close()
