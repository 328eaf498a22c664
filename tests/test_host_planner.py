"""Host logic of libzi.so, on the CPU: exported symbols, plan validation and
closed forms, budget decisions and the ring's timing model.

No call here touches a GPU: zi_plan_tiles, zi_prefetch_depth and
zi_plan_predict are host-only, and the error paths of the pass entry points
return before any HIP call.  Expected values come from the oracle's closed
forms (oracle/closed_forms.py) and the pages' printed numbers.
"""
import ctypes
import math
import os
import re

import pytest

from oracle import closed_forms as cf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def zi():
    from offload_memory_centric_amd import zi as z
    return z


def header_functions():
    text = open(os.path.join(ROOT, "include", "zi.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zi_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_header_function(zi):
    lib = ctypes.CDLL(zi.LIB_PATH)
    names = header_functions()
    assert len(names) >= 19, names
    for n in names:
        assert hasattr(lib, n), "libzi.so does not export %s" % n
    # and the binding wraps exactly those
    assert sorted(zi.EXPORTED) == names
    assert zi.zi_version() >= 100
    assert zi.zi_last_error() == ""


def problem(zi, T=4096, K=8192, M=32768, N=8, d=2, dtype=1, budget=0, dw=True, flags=0):
    return zi.zi_problem(T=T, K=K, M=M, N=N, d=d, dtype=dtype, flags=flags, device_budget_bytes=budget,
                         W_host=None, dW_host=(1 << 20) if dw else None)


def test_plan_info_matches_closed_forms(zi):
    for (T, K, M, N) in [(128, 512, 2048, 4), (4096, 8192, 32768, 8), (4096, 25600, 102400, 16),
                         (2048, 65536, 262144, 16), (32768, 102400, 25600, 16)]:
        _, info = zi.zi_plan_tiles(problem(zi, T, K, M, N), make_plan=False)
        n = cf.tile_cols(M, N)
        assert info.n == n
        assert info.tile_bytes == cf.tile_bytes(K, n)
        assert info.flops_fwd == cf.flops_fwd(T, K, M)
        assert info.flops_bwd == cf.flops_bwd(T, K, M)
        assert info.h2d_bytes_pass == K * M * 2
        assert info.ait_fwd == pytest.approx(cf.link_ait_fwd(T))
        assert info.ait_bwd == pytest.approx(cf.link_ait_bwd(T))
        assert info.working_bytes_one == pytest.approx(cf.working_bytes(K * M * 2, N))
        assert info.working_bytes_two == pytest.approx(cf.working_bytes(K * M * 2, N, in_flight=True))


def test_tiling_examples_of_the_pages(zi):
    # transformer-math page, "Memory-centric tiling": 25600 x 102400, k = 8 -> 655 MB, 1.3 GB
    _, info = zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 8), make_plan=False)
    assert info.tile_bytes == 655_360_000
    assert info.working_bytes_two == pytest.approx(1.31072e9)
    # pwwt.cn article, hd = 64K example: N = 16 tiles of 16K columns, 2 GiB each
    _, info = zi.zi_plan_tiles(problem(zi, 2048, 65536, 262144, 16), make_plan=False)
    assert info.n == 16384 and info.tile_bytes == 2 ** 31


def test_budget_of_two_tiles(zi):
    # 1T-model FFN first matrix, budget capped at two tiles: d = 2 fits with
    # the gradient formed in the weight slot, d = 3 does not fit
    tile = 25600 * 6400 * 2
    _, info = zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 16, d=2, budget=2 * tile), make_plan=False)
    assert info.dw_slots == 0 and info.ring_bytes == 2 * tile
    _, info = zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 16, d=1, budget=2 * tile), make_plan=False)
    assert info.dw_slots == 1 and info.ring_bytes == 2 * tile
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 16, d=3, budget=2 * tile), make_plan=False)
    assert e.value.status == zi.ZI_ERR_BUDGET
    assert "budget" in zi.zi_last_error()
    # no cap: two gradient slots for full-duplex write-back
    _, info = zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 16, d=2), make_plan=False)
    assert info.dw_slots == 2 and info.ring_bytes == 4 * tile
    # forward-only plan: no gradient slots
    _, info = zi.zi_plan_tiles(problem(zi, 4096, 25600, 102400, 16, d=2, dw=False), make_plan=False)
    assert info.dw_slots == 0 and info.ring_bytes == 2 * tile


def test_fp32_gradients_need_their_own_slot(zi):
    tile = 512 * 512 * 2
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_tiles(problem(zi, 128, 512, 2048, 4, d=2, budget=2 * tile, flags=zi.ZI_FLAG_F32_OUT),
                         make_plan=False)
    assert e.value.status == zi.ZI_ERR_BUDGET
    _, info = zi.zi_plan_tiles(problem(zi, 128, 512, 2048, 4, d=2, flags=zi.ZI_FLAG_F32_OUT), make_plan=False)
    assert info.dw_tile_bytes == 2 * info.tile_bytes and info.dw_slots == 2


@pytest.mark.parametrize("kw,status", [
    (dict(M=2048, N=3), "ZI_ERR_SHAPE"),      # N does not divide M
    (dict(K=500), "ZI_ERR_SHAPE"),            # K not a multiple of 8
    (dict(M=2044, N=4), "ZI_ERR_SHAPE"),      # n = 511
    (dict(d=0), "ZI_ERR_ARG"),
    (dict(T=0), "ZI_ERR_SHAPE"),
    (dict(N=0), "ZI_ERR_SHAPE"),
    (dict(dtype=3), "ZI_ERR_ARG"),
    (dict(K=1 << 22), "ZI_ERR_SHAPE"),        # beyond the kernels' 32-bit panel offsets
    (dict(flags=0x10), "ZI_ERR_ARG"),
])
def test_plan_validation(zi, kw, status):
    base = dict(T=128, K=512, M=2048, N=4, d=1, dtype=1)
    base.update(kw)
    p = zi.zi_problem(**base)
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_tiles(p, make_plan=False)
    assert zi.STATUS_NAMES[e.value.status] == status


def test_uneven_but_aligned_split_is_valid(zi):
    _, info = zi.zi_plan_tiles(zi.zi_problem(T=128, K=512, M=2040, N=5, d=1, dtype=1), make_plan=False)
    assert info.n == 408


def test_null_arguments_are_rejected_without_a_gpu(zi):
    lib = ctypes.CDLL(zi.LIB_PATH)
    lib.zi_plan_tiles.argtypes = [ctypes.c_void_p] * 3
    assert lib.zi_plan_tiles(None, None, None) == zi.ZI_ERR_ARG
    for name, nargs in [("zi_tiled_linear_fwd", 4), ("zi_tiled_linear_bwd", 5), ("zi_tiled_linear_fwd_gelu", 5),
                        ("zi_tiled_linear_bwd_recompute", 6), ("zi_sync", 1), ("zi_ctx_stats", 2),
                        ("zi_ctx_timed_records", 4)]:
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_void_p] * nargs
        assert f(*([None] * nargs)) == zi.ZI_ERR_ARG, name
    lib.zi_ctx_create.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_void_p] * 4
    assert lib.zi_ctx_create(None, None, 0, None, None, None, None) == zi.ZI_ERR_ARG
    # the no-allocation forward checks its arguments and the tile against its
    # static buffer before any HIP call (the pointers here are never read)
    lib.zi_tiled_linear_fwd_noalloc.argtypes = [ctypes.c_void_p] * 4
    assert lib.zi_tiled_linear_fwd_noalloc(None, None, None, None) == zi.ZI_ERR_ARG
    big, _ = zi.zi_plan_tiles(zi.zi_problem(T=16, K=8192, M=16400, N=2, d=1, dtype=zi.ZI_F16, flags=0,
                                            device_budget_bytes=0, W_host=None, dW_host=None))
    fake = 1 << 40
    assert lib.zi_tiled_linear_fwd_noalloc(big, None, fake, None) == zi.ZI_ERR_ARG
    assert lib.zi_tiled_linear_fwd_noalloc(big, fake + 8, fake, None) == zi.ZI_ERR_ALIGN
    assert lib.zi_tiled_linear_fwd_noalloc(big, fake, fake, None) == zi.ZI_ERR_BUDGET
    assert "static tile buffer" in zi.zi_last_error()
    fits, _ = zi.zi_plan_tiles(zi.zi_problem(T=16, K=8192, M=8192, N=2, d=1, dtype=zi.ZI_F16, flags=0,
                                             device_budget_bytes=0, W_host=None, dW_host=None))
    assert lib.zi_tiled_linear_fwd_noalloc(fits, fake, fake, None) == zi.ZI_ERR_ARG  # no W_host
    zi.zi_plan_destroy(big)
    zi.zi_plan_destroy(fits)
    lib.zi_stream_create.argtypes = [ctypes.c_void_p]
    assert lib.zi_stream_create(None) == zi.ZI_ERR_ARG
    lib.zi_copy_stream_create.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    out = ctypes.c_void_p()
    assert lib.zi_copy_stream_create(8, None) == zi.ZI_ERR_ARG
    assert lib.zi_copy_stream_create(0, ctypes.byref(out)) == zi.ZI_ERR_ARG
    assert lib.zi_copy_stream_create(-3, ctypes.byref(out)) == zi.ZI_ERR_ARG


def test_prefetch_depth_rule(zi):
    # transformer-math page, "Prefetch depth": 5.2 / 2.05 = 2.5 -> d = 3; striped 0.08 -> d = 1
    assert zi.zi_prefetch_depth(5.2, 2.05) == 3 == cf.prefetch_depth(5.2, 2.05)
    assert zi.zi_prefetch_depth(0.08, 2.05) == 1 == cf.prefetch_depth(0.08, 2.05)
    assert zi.zi_prefetch_depth(4.1, 2.05) == 2
    assert zi.zi_prefetch_depth(0.0, 1.0) == 1
    for tf, tl in [(1.0, 3.0), (10.0, 3.0), (9.0, 3.0), (9.0001, 3.0)]:
        assert zi.zi_prefetch_depth(tf, tl) == cf.prefetch_depth(tf, tl)


# ---- the ring's timing model ------------------------------------------------------

def plan_for_model(zi, N=8, d=2, budget=0):
    p = problem(zi, T=4096, K=8192, M=4096 * N, N=N, d=d, budget=budget)   # tiles of n = 4096
    h, info = zi.zi_plan_tiles(p)
    return h, info


def test_model_depth_one_is_serial(zi):
    h, info = plan_for_model(zi, N=8, d=1)
    tile_flops = 2.0 * 4096 * 8192 * info.n
    R, BW = 1e15, 5e10
    t_c, t_h = tile_flops / R, info.tile_bytes / BW
    pred = zi.zi_plan_predict(h, 0, R, BW, BW)
    assert pred.t_pass_s == pytest.approx(8 * (t_c + t_h))
    assert pred.t_compute_s == pytest.approx(8 * t_c)
    assert pred.stall_frac == pytest.approx(1 - t_c / (t_c + t_h))
    zi.zi_plan_destroy(h)


def test_model_double_buffer_hides_the_faster_stage(zi):
    h, info = plan_for_model(zi, N=8, d=2)
    tile_flops = 2.0 * 4096 * 8192 * info.n
    BW = 5e10
    t_h = info.tile_bytes / BW
    # compute-bound: each tile's product is longer than its copy
    R = tile_flops / (2 * t_h)
    pred = zi.zi_plan_predict(h, 0, R, BW, BW)
    assert pred.t_pass_s == pytest.approx(t_h + 8 * 2 * t_h)   # fill, then compute back to back
    # link-bound: copies back to back, compute hidden except the last tile
    R = tile_flops / (0.5 * t_h)
    pred = zi.zi_plan_predict(h, 0, R, BW, BW)
    assert pred.t_pass_s == pytest.approx(8 * t_h + 0.5 * t_h)
    # pages' depth for the link-bound case: ceil(t_fetch / t_layer) = 2
    assert pred.d_pages == 2 == cf.prefetch_depth(t_h, 0.5 * t_h)
    zi.zi_plan_destroy(h)


def test_model_matches_pipeline_rule(zi):
    # the pipeline runs at the pace of its slowest stage: t_pass -> N * max(t_c, t_h) for large N
    for d in (2, 3):
        h, info = plan_for_model(zi, N=64, d=d)
        tile_flops = 2.0 * 4096 * 8192 * info.n
        for R in (2e14, 2e15):
            BW = 5e10
            t_c, t_h = tile_flops / R, info.tile_bytes / BW
            pred = zi.zi_plan_predict(h, 0, R, BW, BW)
            assert pred.t_pass_s == pytest.approx(64 * max(t_c, t_h) + min(t_c, t_h), rel=1e-9)
        zi.zi_plan_destroy(h)


def test_model_backward_separate_and_in_slot(zi):
    tile = 8192 * 4096 * 2
    R, BW = 1e15, 5e10
    h_sep, info = plan_for_model(zi, N=8, d=2)
    h_in, info_in = plan_for_model(zi, N=8, d=2, budget=2 * tile)
    assert info.dw_slots == 2 and info_in.dw_slots == 0
    sep = zi.zi_plan_predict(h_sep, 1, R, BW, BW)
    ins = zi.zi_plan_predict(h_in, 1, R, BW, BW)
    tile_flops = 2.0 * 4096 * 8192 * info.n
    assert sep.t_compute_s == pytest.approx(8 * 2 * tile_flops / R)
    # with copies faster than products, forming dW in the weight slot can only
    # lengthen the pass (link-bound, the paired dX of separate slots holds two
    # slots and can cost more)
    fast_sep = zi.zi_plan_predict(h_sep, 1, R, 100 * BW, 100 * BW)
    fast_ins = zi.zi_plan_predict(h_in, 1, R, 100 * BW, 100 * BW)
    assert fast_ins.t_pass_s >= fast_sep.t_pass_s - 1e-15
    # recompute adds one product per tile
    rec = zi.zi_plan_predict(h_sep, 2, R, BW, BW)
    assert rec.t_compute_s == pytest.approx(8 * 3 * tile_flops / R)
    with pytest.raises(zi.ZiError):
        zi.zi_plan_predict(h_sep, 4, R, BW, BW)
    zi.zi_plan_destroy(h_sep)
    zi.zi_plan_destroy(h_in)


def test_model_paired_recompute_matches_the_oracle(zi):
    # backward = 3: the recomputed products of a dX pair run once tile 2j + 1
    # has landed.  The library's recurrence against the oracle's, link-bound
    # and compute-bound, with an odd tile count (the last tile on its own).
    for N in (8, 7):
        for BW in (5e10, 5e12):
            R = 1e15
            h, info = plan_for_model(zi, N=N, d=2)
            assert info.dw_slots == 2
            tile_flops = 2.0 * 4096 * 8192 * info.n
            p = {"t_copy": info.tile_bytes / BW, "backward": True, "t_re": tile_flops / R,
                 "t_dx": tile_flops / R, "t_dw": tile_flops / R, "t_back": info.dw_tile_bytes / BW}
            for bwd, extra in ((2, {}), (3, {"re_pairs": True})):
                got = zi.zi_plan_predict(h, bwd, R, BW, BW)
                want = cf.ring_run(N, 2, [dict(p, pairs=True, **extra)], grad_slots=2)[0]
                assert got.t_pass_s == pytest.approx(want, rel=1e-12), (N, BW, bwd)
                assert got.t_compute_s == pytest.approx(N * 3 * tile_flops / R)
            zi.zi_plan_destroy(h)


# --- tile-width choice: zi_plan_choose against the oracle's brute force ------

def _problem(zi, T, K, M, dtype, budget, f32=False):
    return zi.zi_problem(T=T, K=K, M=M, N=1, d=1, dtype=zi.DTYPE_CODES[dtype],
                         flags=zi.ZI_FLAG_F32_OUT if f32 else 0, device_budget_bytes=budget,
                         W_host=None, dW_host=None)


def _same(got, want):
    for k in ("N", "d", "n", "dw_slots", "ring_bytes"):
        assert got[k] == want[k], (k, got, want)
    # the two recurrences group a few sums differently: equal to rounding
    for k in ("t_fwd_s", "t_bwd_s", "t_step_s"):
        assert got[k] == pytest.approx(want[k], rel=1e-10, abs=0.0), (k, got, want)


@pytest.mark.parametrize("seed", range(40))
def test_choice_matches_the_oracle(zi, seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    dtype = ["f16", "bf16"][seed % 2]
    f32 = seed % 5 == 0
    K = int(rng.choice([1024, 4096, 8192, 25600]))
    M = int(rng.choice([8192, 32768, 102400, 25600 * 3]))
    T = int(rng.choice([256, 4096, 32768]))
    divs = [n for n in range(8, M + 1, 8) if M % n == 0]
    widths = sorted(set(int(x) for x in rng.choice(divs, size=min(len(divs), 6), replace=False)))
    widths.append(widths[-1] + 4)  # a width that does not divide M
    base = rng.uniform(5e14, 1.5e15)
    fwd = [base * n / (n + rng.uniform(100, 3000)) for n in widths]
    dx = [r * rng.uniform(0.8, 1.1) for r in fwd]
    dw = [r * rng.uniform(0.8, 1.1) for r in fwd]
    h2d, d2h = rng.uniform(2e10, 6e10), rng.uniform(2e10, 6e10)
    backward = int(seed % 4)
    max_d = int(rng.integers(1, 5))
    tile_max = K * widths[-2] * 2
    budget = 0 if seed % 4 == 0 else int(rng.uniform(1.0, 5.0) * tile_max)
    # half the cases carry copy rates per width (small copies run slower)
    c_h2d = [h2d * n / (n + 500) for n in widths] if seed % 2 else None
    c_d2h = [d2h * n / (n + 900) for n in widths] if seed % 2 else None
    want, table = cf.choose_tiling(T, K, M, dtype, budget, widths, fwd, dx, dw, h2d, d2h, backward, max_d,
                                   grad_f32=f32, c_h2d=c_h2d, c_d2h=c_d2h)
    if want is None:
        with pytest.raises(zi.ZiError) as e:
            zi.zi_plan_choose(_problem(zi, T, K, M, dtype, budget, f32), widths, fwd, dx, dw, h2d, d2h,
                              backward, max_d, h2d=c_h2d, d2h=c_d2h)
        assert e.value.status == zi.ZI_ERR_BUDGET
        return
    got, got_table = zi.zi_plan_choose(_problem(zi, T, K, M, dtype, budget, f32), widths, fwd, dx, dw,
                                       h2d, d2h, backward, max_d, h2d=c_h2d, d2h=c_d2h)
    _same(got, want)
    assert len(got_table) == len(table)
    for g, w in zip(got_table, table):
        _same(g, w)


def test_choice_agrees_with_plan_predict(zi):
    # the chosen candidate's forward time is what zi_plan_predict gives the
    # same plan at the same rate and link rate
    T, K, M = 4096, 8192, 32768
    widths = [1024, 2048, 4096, 8192]
    fwd = [1e15] * 4
    got, table = zi.zi_plan_choose(_problem(zi, T, K, M, "bf16", 0), widths, fwd, None, None, 5e10, 5e10,
                                   1, 3)
    for c in table:
        prob = zi.zi_problem(T=T, K=K, M=M, N=c["N"], d=c["d"], dtype=zi.ZI_BF16, flags=0,
                             device_budget_bytes=0, W_host=None, dW_host=1 << 12)
        h, info = zi.zi_plan_tiles(prob)
        try:
            assert info.ring_bytes == c["ring_bytes"]
            assert zi.zi_plan_predict(h, 0, 1e15, 5e10, 5e10).t_pass_s == pytest.approx(c["t_fwd_s"], rel=1e-14)
            assert zi.zi_plan_predict(h, 1, 1e15, 5e10, 5e10).t_pass_s == pytest.approx(c["t_bwd_s"], rel=1e-14)
        finally:
            zi.zi_plan_destroy(h)


def test_choice_errors(zi):
    T, K, M = 4096, 8192, 32768
    p = _problem(zi, T, K, M, "f16", 0)
    with pytest.raises(zi.ZiError) as e:  # no width divides M
        zi.zi_plan_choose(p, [3000, 5000], [1e15, 1e15], h2d_bytes_per_s=5e10, d2h_bytes_per_s=5e10)
    assert e.value.status == zi.ZI_ERR_SHAPE
    with pytest.raises(zi.ZiError) as e:  # nothing fits
        zi.zi_plan_choose(_problem(zi, T, K, M, "f16", 4096), [4096], [1e15], h2d_bytes_per_s=5e10,
                          d2h_bytes_per_s=5e10)
    assert e.value.status == zi.ZI_ERR_BUDGET
    for bad in (dict(fwd=[0.0]), dict(fwd=[float("nan")]), dict(fwd=[1e15], dx=[-1.0])):
        kw = dict(fwd=[1e15])
        kw.update(bad)
        with pytest.raises(zi.ZiError) as e:
            zi.zi_plan_choose(p, [4096], h2d_bytes_per_s=5e10, d2h_bytes_per_s=5e10, **kw)
        assert e.value.status == zi.ZI_ERR_ARG
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_choose(p, [4096], [1e15], h2d_bytes_per_s=0.0, d2h_bytes_per_s=5e10)
    assert e.value.status == zi.ZI_ERR_ARG
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_choose(p, [4096], [1e15], h2d_bytes_per_s=5e10, d2h_bytes_per_s=5e10, max_d=0)
    assert e.value.status == zi.ZI_ERR_ARG
    with pytest.raises(zi.ZiError) as e:
        zi.zi_plan_choose(p, [4096], [1e15], h2d_bytes_per_s=5e10, d2h_bytes_per_s=5e10, backward=4)
    assert e.value.status == zi.ZI_ERR_ARG
    with pytest.raises(zi.ZiError) as e:  # the problem's own shape
        zi.zi_plan_choose(_problem(zi, T, 8190, M, "f16", 0), [4096], [1e15], h2d_bytes_per_s=5e10,
                          d2h_bytes_per_s=5e10)
    assert e.value.status == zi.ZI_ERR_SHAPE


def test_macro_tile_choice(zi):
    # 320-wide workgroup tiles where the tile width is a multiple of 320 but not
    # of 256 (the down-projection's 1600-column tiles: 5 tiles of 320 against
    # 6.25 of 256); 256 x 256 wherever that pads less
    def tiles(T, K, M, N):
        _, info = zi.zi_plan_tiles(zi.zi_problem(T=T, K=K, M=M, N=N, d=2, dtype=zi.ZI_F16, flags=0,
                                                 device_budget_bytes=0, W_host=None, dW_host=None), False)
        return tuple(info.fwd_tile), tuple(info.dw_tile)
    assert tiles(32768, 102400, 25600, 16) == ((192, 320), (320, 192))  # down-projection, n = 1600
    assert tiles(8192, 102400, 25600, 16) == ((192, 320), (320, 192))
    assert tiles(32768, 25600, 102400, 16) == ((256, 256), (256, 256))  # up-projection, n = 6400
    assert tiles(4096, 8192, 32768, 8) == ((256, 256), (256, 256))      # n = 4096
    assert tiles(4096, 25600, 102400, 16) == ((256, 256), (256, 256))
    assert tiles(2048, 65536, 262144, 16) == ((256, 256), (256, 256))
    assert tiles(380, 584, 3200, 2) == ((192, 320), (320, 192))
    assert tiles(7200, 128, 1600, 1) == ((192, 320), (320, 192))
