"""GPU parity of the tiled linear operator against the oracle (small shapes).

Every case runs the library through its C ABI (binding in
offload_memory_centric_amd.zi) and compares with the oracle element by element.
"""
import numpy as np
import pytest
import torch

import oracle
from offload_memory_centric_amd import inputs
from zi_testlib import (assert_close, host_bits, lib, make_linear_inputs, say, values)

pytestmark = pytest.mark.gpu


def run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY, f32_out=False, budget=0, want_bwd=True, **ctx_kw):
    tiling = lib()
    elem = torch.float32 if f32_out else inputs.torch_dtype(dtype)
    dWt = tiling.host_tensor((M, K), elem) if want_bwd else None
    plan = tiling.Plan(T, K, M, N, d, dtype, Wt, dWt, budget=budget, f32_out=f32_out)
    ctx = tiling.Context(plan, **ctx_kw)
    Y = torch.empty((T, M), dtype=elem, device="cuda")
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y)
    if want_bwd:
        ctx.bwd(plan, X, dY, dX)
    ctx.sync()
    out = {"Y": Y, "dX": dX, "dWt": dWt, "info": plan.info}
    ctx.close()
    plan.close()
    return out


def oracle_linear(X, Wt, dY, dtype):
    Xb, Wb, dYb = host_bits(X), host_bits(Wt), host_bits(dY)
    Y = oracle.linear_fwd(Xb, Wb, dtype)
    dX, dWt = oracle.linear_bwd(Xb, Wb, dYb, dtype)
    return Y, dX, dWt


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,d", [(4, 1), (4, 2), (2, 1), (2, 2), (1, 1), (1, 2)])
def test_small_integers_bit_exact(dtype, N, d):
    # X[128x512], W[512x2048], dY[128x2048] with values in {-3..3}: every fp32
    # partial sum is an integer below 2^24, so sums are exact in any order and
    # one RNE makes the stored results unique.
    T, K, M = 128, 512, 2048
    say("case small_int", dtype, "N", N, "d", d)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=0)
    r = run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, dtype)
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, dtype)), "Y bits"
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX), "dX exact"
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, dtype)), "dW bits"


@pytest.mark.parametrize("d", [1, 2])
def test_gaussian_f16(d):
    T, K, M, N = 128, 512, 2048, 4
    say("case gaussian f16 d", d)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "gaussian", seed=0)
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    assert_close(values(r["Y"], "f16"), Y, "Y")
    assert_close(values(r["dX"], "f16"), dX, "dX")
    assert_close(values(r["dWt"], "f16"), dWt, "dW")


def test_gaussian_bf16_fp32_epilogue_and_rounding():
    # bf16's own half-ulp near max|Y| is above 2e-3 * max|Y|, so the tolerance
    # is checked on the kernel's fp32 epilogue; the bf16 results must then be
    # exactly one RNE rounding of those fp32 values.
    T, K, M, N, d = 128, 512, 2048, 4, 2
    say("case gaussian bf16")
    X, Wt, dY = make_linear_inputs(T, K, M, "bf16", "gaussian", seed=1)
    r32 = run_fwd_bwd(T, K, M, N, d, "bf16", X, Wt, dY, f32_out=True)
    r16 = run_fwd_bwd(T, K, M, N, d, "bf16", X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "bf16")
    assert_close(values(r32["Y"], "bf16"), Y, "Y(fp32)")
    assert_close(values(r32["dX"], "bf16"), dX, "dX")
    assert_close(values(r32["dWt"], "bf16"), dWt, "dW(fp32)")
    assert torch.equal(r16["Y"].cpu(), r32["Y"].cpu().to(torch.bfloat16)), "Y16 != RNE(Y32)"
    assert torch.equal(r16["dWt"], r32["dWt"].to(torch.bfloat16)), "dW16 != RNE(dW32)"
    assert torch.equal(r16["dX"], r32["dX"]), "dX differs between epilogues"
    # raw bf16 vs oracle: within one bf16 ulp of the largest value
    err = np.abs(values(r16["Y"], "bf16") - Y).max()
    say("  raw bf16 Y max|err| %.3e (max|ref| %.3e)" % (err, np.abs(Y).max()))
    assert err <= 2.0 ** -7 * np.abs(Y).max()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ragged_shapes(dtype):
    # several macro-tiles with ragged tails in every dimension:
    # T = 300 (256 + 44), K = 520 (not a multiple of 64), n = 200 (< 256)
    T, K, M, N, d = 300, 520, 600, 3, 2
    say("case ragged", dtype)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "gaussian", seed=2)
    r = run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY, f32_out=True)
    Y, dX, dWt = oracle_linear(X, Wt, dY, dtype)
    assert_close(values(r["Y"], dtype), Y, "Y")
    assert_close(values(r["dX"], dtype), dX, "dX")
    assert_close(values(r["dWt"], dtype), dWt, "dW")


def test_ragged_integers_bit_exact():
    T, K, M, N, d = 77, 264, 1040, 5, 2       # n = 208
    say("case ragged small_int")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=3)
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, "f16"))
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX)
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, "f16"))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,M,N,d", [(192, 320, 576, 3, 2), (64, 192, 576, 1, 1), (128, 64, 384, 6, 2)])
def test_odd_step_counts_bit_exact(dtype, T, K, M, N, d):
    # reduction lengths that are multiples of the 64-value step but an odd
    # number of steps (forward K, dW T, dX n, and the paired dX 2n), where the
    # main loop runs one step past the end on zero fragments
    say("case odd steps", dtype, T, K, M, N, d)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=11)
    r = run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, dtype)
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, dtype)), "Y bits"
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX), "dX exact"
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, dtype)), "dW bits"


def test_minimum_shapes():
    T, K, M, N, d = 1, 8, 8, 1, 1
    say("case minimum")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=4)
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, "f16"))
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX)
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, "f16"))


def test_ramp_column_offsets():
    # X rows = e_0 and W[0][m] = m mod 2048: Y[t][m] = m mod 2048 exactly, which
    # exposes any misplaced tile or column.
    T, K, M, N, d = 64, 64, 4096, 8, 2
    say("case ramp")
    tiling = lib()
    X = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    X[:, 0] = 1
    Wt = tiling.host_tensor((M, K), torch.float16)
    Wt.zero_()
    Wt[:, 0] = torch.arange(M, dtype=torch.float32).remainder(2048).to(torch.float16)
    dY = torch.zeros((T, M), dtype=torch.float16, device="cuda")
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    expect = np.tile(np.arange(M) % 2048, (T, 1)).astype(np.float64)
    assert np.array_equal(values(r["Y"], "f16"), expect)


def test_fp16_subnormal_weights():
    # W entries are fp16 subnormals k * 2^-24; X small integers: every product
    # and sum is exact in fp32, so the result shows whether subnormal operands
    # are honoured by the matrix cores.
    T, K, M, N, d = 64, 128, 256, 2, 1
    say("case subnormal")
    tiling = lib()
    X = inputs.new((T, K), "f16", "small_int", 5, "X", device="cuda")
    Wt = tiling.host_tensor((M, K), torch.float16)
    g = torch.Generator().manual_seed(5)
    k = torch.randint(-1023, 1024, (M, K), generator=g, dtype=torch.int32)
    Wt.view(torch.int16).copy_((k.abs() | (k < 0).to(torch.int32) * 0x8000).to(torch.int16))
    dY = inputs.new((T, M), "f16", "small_int", 5, "dY", device="cuda")
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY, f32_out=True)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    got = values(r["Y"], "f16")
    say("  subnormal Y max|ref| %.3e max|got| %.3e" % (np.abs(Y).max(), np.abs(got).max()))
    assert np.array_equal(got, Y)
    assert np.array_equal(values(r["dX"], "f16"), dX)


def test_results_independent_of_N_and_d():
    # per-element reduction order over K (Y) and over T (dW) does not depend on
    # the tile width, so Y and dW are bit-identical for any N and d
    T, K, M = 256, 1024, 2048
    say("case invariance")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "gaussian", seed=6)
    base = run_fwd_bwd(T, K, M, 1, 1, "f16", X, Wt, dY)
    for N, d in [(2, 1), (4, 2), (8, 3)]:
        r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
        assert torch.equal(r["Y"], base["Y"]), (N, d)
        assert torch.equal(r["dWt"], base["dWt"]), (N, d)
        err = (r["dX"] - base["dX"]).abs().max().item()
        assert err <= 1e-4 * base["dX"].abs().max().item(), (N, d, err)


def test_gradient_in_weight_slot_matches_separate_slots():
    T, K, M, N, d = 128, 512, 2048, 4, 2
    say("case in-slot gradients")
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "gaussian", seed=7)
    tile = K * (M // N) * 2
    sep = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    ins = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY, budget=d * tile)
    assert sep["info"].dw_slots == 2 and ins["info"].dw_slots == 0
    assert torch.equal(sep["Y"], ins["Y"])
    assert torch.equal(sep["dWt"], ins["dWt"])
    # with separate gradient slots the dX products of tiles 2j, 2j+1 are one
    # launch, so dX is summed in another order: equal up to fp32 rounding
    err = (sep["dX"] - ins["dX"]).abs().max().item()
    assert err <= 1e-5 * ins["dX"].abs().max().item(), err


@pytest.mark.parametrize("h2d_cus,d2h_cus", [(8, 0), (8, 8), (8, 32), (0, 8), (16, 16)])
def test_copy_stream_confinement(h2d_cus, d2h_cus):
    # the tile copy and dW write-back streams confined to 8, 16 or 32 compute
    # units, or unconfined (0): the same exact results
    T, K, M, N, d = 128, 512, 2048, 4, 2
    say("case copy stream cus", h2d_cus, d2h_cus)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=6)
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY, h2d_cus=h2d_cus, d2h_cus=d2h_cus)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, "f16"))
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX)
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, "f16"))


def test_copy_stream_cu_count_checked():
    from offload_memory_centric_amd import zi
    say("case copy stream n_cus range")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for bad in (0, -1, 1, 12, cus + 8):
        with pytest.raises(zi.ZiError) as e:
            zi.zi_copy_stream_create(bad)
        assert e.value.status == zi.ZI_ERR_ARG
    for good in (8, cus):
        s = zi.zi_copy_stream_create(good)
        zi.zi_stream_destroy(s)


@pytest.mark.parametrize("N,d", [(3, 2), (5, 3), (6, 2)])
def test_paired_dx_odd_and_even_tile_counts(N, d):
    # n = 512 (a multiple of the kernel step): dX of tile pairs in one launch,
    # an odd last tile alone; small integers keep every result exact
    T, K, n = 128, 512, 512
    M = N * n
    say("case paired dX N", N, "d", d)
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=11)
    r = run_fwd_bwd(T, K, M, N, d, "f16", X, Wt, dY)
    assert r["info"].dw_slots == 2
    Y, dX, dWt = oracle_linear(X, Wt, dY, "f16")
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, "f16"))
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX)
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, "f16"))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,M,N,d", [(2304, 20480, 512, 4, 2), (1100, 14000, 600, 3, 2)])
def test_persistent_dx_bit_exact(dtype, T, K, M, N, d):
    # dX with more 256 x 256 output blocks than the compute units' persistent
    # workgroups: 9 x 80 = 720 blocks (about three per workgroup, tile pairs:
    # an aligned reduction of 256 over two slots, the first pair overwriting,
    # the second adding), and 5 x 55 = 275 (ragged rows and columns, unpaired
    # tiles of 200: an unaligned reduction).  Small integers make dX exact;
    # the per-block form must give the same bits.
    tiling = lib()
    say("case persistent dX", dtype, "T", T, "K", K, "M", M, "N", N, "d", d)
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=23)
    outs = []
    dWt = tiling.host_tensor((M, K), inputs.torch_dtype(dtype))
    for per_tile in (False, True):
        plan = tiling.Plan(T, K, M, N, d, dtype, Wt, dWt)
        ctx = tiling.Context(plan)
        ctx.set_debug(dx_per_tile=per_tile)
        dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        ctx.bwd(plan, X, dY, dX)
        ctx.sync()
        outs.append(dX.cpu().numpy())
        ctx.close()
        plan.close()
    ref, ref_dw = oracle.linear_bwd(host_bits(X), host_bits(Wt), host_bits(dY), dtype)
    assert np.array_equal(outs[0].astype(np.float64), ref), "persistent dX against the oracle"
    assert np.array_equal(host_bits(dWt), oracle.encode(ref_dw, dtype)), "dW bits"
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "persistent against per-block dX"


@pytest.mark.parametrize("dtype,K", [("f16", 4608), ("bf16", 256)])
def test_banded_and_grouped_tile_orders_bit_exact(dtype, K):
    # T = 4096: 16 macro-rows of 256, one whole band, so the forward and dX
    # take their tiles in the band order (XCD pairs on 4-row strips); the
    # tile of 2600 makes 11 dW row tiles, one 8-row group that all XCDs walk
    # together and 3 rows split by ranges.  K = 4608: 16 x 18 = 288 dX blocks,
    # more than the persistent workgroups.  Small integers: Y, dX and dW
    # unique (|Y| <= 9 K, |dX| <= 9 M, |dW| <= 9 T, all within fp16's range).
    T, M, N, d = 4096, 2600, 1, 1
    say("case tile orders", dtype, T, K, M, N, d)
    tiling = lib()
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=31)
    info = tiling.Plan(T, K, M, N, d, dtype, None).info
    assert tuple(info.fwd_tile) == (256, 256) and tuple(info.dw_tile) == (256, 256)
    r = run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, dtype)
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, dtype)), "Y bits"
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX), "dX exact"
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, dtype)), "dW bits"


def test_consecutive_calls_share_the_ring():
    # two forwards and a backward enqueued back to back with no host sync:
    # the first copies of each call overlap the previous call's products
    T, K, M, N, d = 128, 512, 2048, 4, 2
    say("case cross-call")
    tiling = lib()
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "small_int", seed=8)
    X2 = inputs.new((T, K), "f16", "small_int", 9, "X", device="cuda")
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, dWt)
    ctx = tiling.Context(plan)
    Y1 = torch.empty((T, M), dtype=torch.float16, device="cuda")
    Y2 = torch.empty_like(Y1)
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y1)
    ctx.fwd(plan, X2, Y2)
    ctx.bwd(plan, X, dY, dX)
    ctx.fwd(plan, X, Y1)
    ctx.sync()
    Y, dXr, dWr = oracle_linear(X, Wt, dY, "f16")
    Y2r = oracle.linear_fwd(host_bits(X2), host_bits(Wt), "f16")
    assert np.array_equal(host_bits(Y1), oracle.encode(Y, "f16"))
    assert np.array_equal(host_bits(Y2), oracle.encode(Y2r, "f16"))
    assert np.array_equal(dX.cpu().numpy().astype(np.float64), dXr)
    assert np.array_equal(host_bits(dWt), oracle.encode(dWr, "f16"))
    ctx.close()
    plan.close()


@pytest.mark.parametrize("T,K,M,N,d", [(200, 512, 1536, 3, 2), (700, 576, 3200, 2, 2)])
def test_recompute_matches_forward_bit_for_bit(T, K, M, N, d):
    # (700, 576, 3200): tiles of 1600 in 192 x 320 workgroup tiles, so the
    # recompute of the pair is one launch of 10 tile columns (the first tile's
    # five on XCDs 0-3, the second's on 4-7) against five per forward launch
    say("case recompute", T, K, M, N, d)
    tiling = lib()
    X, Wt, dY = make_linear_inputs(T, K, M, "f16", "gaussian", seed=10)
    dWt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt, dWt)
    ctx = tiling.Context(plan)
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    Yr = torch.empty_like(Y)
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dX2 = torch.empty_like(dX)
    torch.cuda.synchronize()
    ctx.fwd(plan, X, Y)
    ctx.bwd_recompute(plan, X, dY, dX, Yr)
    ctx.sync()
    dW1 = dWt.clone()
    ctx.bwd(plan, X, dY, dX2)
    ctx.sync()
    assert torch.equal(Y, Yr)
    assert torch.equal(dX, dX2)
    assert torch.equal(dW1, dWt)
    Yo, dXo, dWo = oracle_linear(X, Wt, dY, "f16")
    assert_close(values(Y, "f16"), Yo, "Y")
    assert_close(values(dX, "f16"), dXo, "dX")
    assert_close(values(dWt, "f16"), dWo, "dW")
    ctx.close()
    plan.close()


# ---- error paths ----------------------------------------------------------------

def test_budget_error_and_in_slot_choice():
    from offload_memory_centric_amd import zi
    tiling = lib()
    T, K, M, N = 64, 256, 1024, 4
    tile = K * (M // N) * 2
    Wt = tiling.host_tensor((M, K), torch.float16)
    dWt = tiling.host_tensor((M, K), torch.float16)
    with pytest.raises(zi.ZiError) as e:
        tiling.Plan(T, K, M, N, 3, "f16", Wt, dWt, budget=2 * tile)
    assert e.value.status == zi.ZI_ERR_BUDGET
    p = tiling.Plan(T, K, M, N, 2, "f16", Wt, dWt, budget=2 * tile)
    assert p.info.dw_slots == 0 and p.info.ring_bytes == 2 * tile
    # fp32 gradients cannot live in a 16-bit weight slot
    with pytest.raises(zi.ZiError) as e:
        tiling.Plan(T, K, M, N, 2, "f16", Wt, dWt, budget=2 * tile, f32_out=True)
    assert e.value.status == zi.ZI_ERR_BUDGET


def test_unpinned_weights_rejected():
    from offload_memory_centric_amd import zi
    tiling = lib()
    T, K, M, N, d = 64, 256, 1024, 4, 2
    Wt = torch.zeros((M, K), dtype=torch.float16)  # pageable
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt)
    ctx = tiling.Context(plan)
    X = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    with pytest.raises(zi.ZiError) as e:
        ctx.fwd(plan, X, Y)
    assert e.value.status == zi.ZI_ERR_NOT_PINNED
    ctx.close()


def test_misaligned_pointer_rejected():
    from offload_memory_centric_amd import zi
    tiling = lib()
    T, K, M, N, d = 64, 256, 1024, 4, 2
    Wt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt)
    ctx = tiling.Context(plan)
    X = torch.zeros((T * K + 8,), dtype=torch.float16, device="cuda")
    Y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    with pytest.raises(zi.ZiError) as e:
        zi.zi_tiled_linear_fwd(ctx.handle, plan.handle, X.data_ptr() + 2, Y)
    assert e.value.status == zi.ZI_ERR_ALIGN
    ctx.sync()
    ctx.close()


def test_small_workspace_rejected():
    from offload_memory_centric_amd import zi
    tiling = lib()
    T, K, M, N, d = 64, 256, 1024, 4, 2
    Wt = tiling.host_tensor((M, K), torch.float16)
    plan = tiling.Plan(T, K, M, N, d, "f16", Wt)
    with pytest.raises(zi.ZiError) as e:
        tiling.Context(plan, workspace_bytes=plan.info.ring_bytes - 256)
    assert e.value.status == zi.ZI_ERR_BUDGET


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,M,N,d,fwd_rows", [(380, 584, 3200, 2, 2, 192), (700, 576, 1920, 2, 1, 192),
                                                (32, 1600, 1600, 1, 1, 192), (7200, 128, 1600, 1, 1, 192),
                                                (700, 576, 1280, 2, 2, 192)])
def test_320_wide_tiles_bit_exact(dtype, T, K, M, N, d, fwd_rows):
    # tile widths that 320 divides and 256 does not: the forward runs 192 x 320
    # workgroup tiles, the gradient 320 x 192 (both checked in the
    # plan), with ragged rows (T = 380, 700, 7200), a reduction that is not a
    # multiple of the 64-value step (K = 584, T = 380, 7200) or an odd number
    # of steps (K = 576: 9); small integers, so every result is unique
    # (|dW| <= 9 T stays below fp16's 65504); M = 1280: two tile columns of
    # 320, which the forward takes left half first
    say("case 320-wide tiles", dtype, T, K, M, N, d)
    tiling = lib()
    X, Wt, dY = make_linear_inputs(T, K, M, dtype, "small_int", seed=13)
    info = tiling.Plan(T, K, M, N, d, dtype, None).info
    assert tuple(info.fwd_tile) == (fwd_rows, 320) and tuple(info.dw_tile) == (320, 192)
    r = run_fwd_bwd(T, K, M, N, d, dtype, X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, dtype)
    assert np.array_equal(host_bits(r["Y"]), oracle.encode(Y, dtype)), "Y bits"
    assert np.array_equal(r["dX"].cpu().numpy().astype(np.float64), dX), "dX exact"
    assert np.array_equal(host_bits(r["dWt"]), oracle.encode(dWt, dtype)), "dW bits"


def test_320_wide_tiles_gaussian_bf16():
    # the same shapes on Gaussian values: the fp32 epilogues at the 2e-3 bar
    # and the bf16 results one RNE rounding of them
    T, K, M, N, d = 380, 584, 3200, 2, 2
    say("case 320-wide tiles gaussian bf16")
    X, Wt, dY = make_linear_inputs(T, K, M, "bf16", "gaussian", seed=14)
    r32 = run_fwd_bwd(T, K, M, N, d, "bf16", X, Wt, dY, f32_out=True)
    r16 = run_fwd_bwd(T, K, M, N, d, "bf16", X, Wt, dY)
    Y, dX, dWt = oracle_linear(X, Wt, dY, "bf16")
    assert_close(values(r32["Y"], "bf16"), Y, "Y fp32")
    assert_close(values(r32["dX"], "bf16"), dX, "dX")
    assert_close(values(r32["dWt"], "bf16"), dWt, "dW fp32")
    assert torch.equal(r16["Y"], r32["Y"].to(torch.bfloat16))
    assert torch.equal(r16["dWt"], r32["dWt"].to(torch.bfloat16))
    assert torch.equal(r16["dX"], r32["dX"])
