"""The no-allocation forward (zi_tiled_linear_fwd_noalloc) through the C ABI:
bit-identical to the context's forward (zi_tiled_linear_fwd, the same kernel
and tile order) on two calls in a row, the first with a tile of exactly the
static buffer's size, the second smaller; a larger tile is refused."""
import pytest
import torch

from zi_testlib import lib, make_linear_inputs, say

pytestmark = pytest.mark.gpu


def context_forward(tiling, plan, X, T, M, dtype):
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=X.dtype, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y)
    ctx.sync()
    ctx.close()
    return Y


def test_noalloc_forward_equals_the_context_forward():
    from offload_memory_centric_amd import zi
    tiling = lib()
    stream = torch.cuda.Stream()
    # (T, K, M, N): a tile of K * M/N * 2 bytes = exactly the buffer's 64 MiB,
    # then a smaller, ragged one (T and n not multiples of the 256 macro-tile)
    cases = [(512, 8192, 8192, 2, "bf16", 80), (300, 1024, 4000, 4, "f16", 81)]
    for T, K, M, N, dtype, seed in cases:
        say("case no-alloc forward", T, K, M, N, dtype)
        X, Wt, _ = make_linear_inputs(T, K, M, dtype, "gaussian", seed)
        plan = tiling.Plan(T, K, M, N, 2, dtype, Wt)
        assert plan.info.tile_bytes <= zi.ZI_NOALLOC_SCRATCH_BYTES
        want = context_forward(tiling, plan, X, T, M, dtype)
        got = torch.full_like(want, float("nan"))
        torch.cuda.synchronize()
        zi.zi_tiled_linear_fwd_noalloc(plan.handle, X, got, stream)
        stream.synchronize()
        assert torch.equal(got, want), "no-alloc forward differs from the context's"
        plan.close()
    assert cases[0][1] * (cases[0][2] // cases[0][3]) * 2 == zi.ZI_NOALLOC_SCRATCH_BYTES

    # a tile larger than the buffer is refused before anything runs
    big = tiling.Plan(16, 8192, 8200 * 2, 2, 1, "f16", None)
    X = torch.zeros((16, 8192), dtype=torch.float16, device="cuda")
    Y = torch.zeros((16, 8200 * 2), dtype=torch.float16, device="cuda")
    with pytest.raises(zi.ZiError) as e:
        zi.zi_tiled_linear_fwd_noalloc(big.handle, X, Y, stream)
    assert e.value.status == zi.ZI_ERR_BUDGET
    big.close()
