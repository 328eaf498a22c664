"""The extreme-width layer at its full size (hd = 65536 -> 262144), on sampled
outputs against the oracle.  Its weight and gradient take 64 GiB of pinned host
memory, about what one process on the test host can pin; it sits in a file of
its own that sorts before every other GPU test, so that it runs before any
other test has pinned (and the runtime has kept) host memory."""
import pytest

from test_gpu_configs import big_linear, release_pinned, run_pass, sampled_parity
from zi_testlib import say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_extreme_width_layer():
    # hd = 65536 -> 262144: W and dW 32 GiB each in pinned host memory,
    # N = 16 tiles of 2 GiB, T = 2048, d = 2
    T, K, M, N, d = 2048, 65536, 262144, 16, 2
    say("case extreme width: allocating 64 GiB pinned")
    release_pinned()
    from offload_memory_centric_amd import zi
    try:
        X, Wt, dY = big_linear(T, K, M, N, d, "f16", seed=2, chunk_rows=8192)
        Y, dX, dWt, info = run_pass(T, K, M, N, d, "f16", X, Wt, dY)
    except zi.ZiError as e:
        if "out of memory" in str(e):
            pytest.skip("the host could not pin 64 GiB for W and dW (%s)" % e)
        raise
    assert info.tile_bytes == 2 ** 31
    say("case extreme width: sampled parity")
    sampled_parity(T, K, M, N, "f16", X, Wt, dY, Y, dX, dWt, seed=300)
