"""The oracle's ring timing and tile-width choice, pinned to closed forms and
hand-worked timelines (the pages fix the trade-off, not a formula: resident
bytes fall as layer bytes / k while finer tiles make slower products, and
copies overlap products).  CPU only."""
import pytest

from oracle import closed_forms as cf


def test_forward_pass_closed_forms():
    # d = 1: nothing overlaps
    assert cf.ring_pass_time(5, 1, 2.0, t_fwd=3.0) == 5 * (2.0 + 3.0)
    # d >= 2, copies faster than products: the first copy, then back-to-back products
    for d in (2, 3, 7):
        assert cf.ring_pass_time(6, d, 1.0, t_fwd=3.0) == 1.0 + 6 * 3.0
    # d >= 2, copies slower: back-to-back copies, then the last product
    for d in (2, 4):
        assert cf.ring_pass_time(6, d, 3.0, t_fwd=1.0) == 6 * 3.0 + 1.0


def test_forward_timeline_by_hand():
    # N = 3, d = 2, copy 2, product 1: copies [0,2] [2,4] [4,6] (tile 2's slot
    # is free at 3), products [2,3] [4,5] [6,7]
    assert cf.ring_pass_time(3, 2, 2.0, t_fwd=1.0) == 7.0
    # d = 2 with a slow first product: N = 3, copy 1, product 4: copies
    # [0,1] [1,2]; tile 2 waits for tile 0's slot (free at 5): [5,6];
    # products [1,5] [5,9] [9,13]
    assert cf.ring_pass_time(3, 2, 1.0, t_fwd=4.0) == 13.0


def test_backward_gradient_in_weight_slot_by_hand():
    # N = 3, d = 2, every stage 1, no gradient slot: tile 0 copy [0,1] dX [1,2]
    # dW [2,3] write-back [3,4] (slot free at 4); tile 1 copy [1,2] dX [3,4]
    # dW [4,5] write-back [5,6]; tile 2 copy waits for slot 0: [4,5], dX [5,6]
    # dW [6,7] write-back [7,8]
    assert cf.ring_pass_time(3, 2, 1.0, backward=True, t_dx=1.0, t_dw=1.0, t_back=1.0) == 8.0
    # d = 1: serial
    assert cf.ring_pass_time(4, 1, 1.0, backward=True, t_dx=2.0, t_dw=3.0, t_back=0.5) == 4 * 6.5


def test_backward_with_gradient_slots_closed_form():
    # free write-back and fast copies: one copy, then dX + dW per tile back to back
    for d, g in ((2, 1), (2, 2), (3, 2)):
        t = cf.ring_pass_time(8, d, 0.5, backward=True, t_dx=1.0, t_dw=2.0, t_back=0.0, grad_slots=g)
        assert t == 0.5 + 8 * 3.0
    # with the recompute: it reads the weight slot before dX
    t = cf.ring_pass_time(8, 2, 0.5, backward=True, t_re=1.0, t_dx=1.0, t_dw=1.0, grad_slots=2)
    assert t == 0.5 + 8 * 3.0
    # write-back slower than the products.  One gradient slot: dW_i waits for
    # the write-back of tile i - 1, and its own write-back for dW_i, so each
    # tile costs dW + write-back after the first dX
    t = cf.ring_pass_time(5, 2, 0.1, backward=True, t_dx=1.0, t_dw=1.0, t_back=4.0, grad_slots=1)
    assert t == pytest.approx(0.1 + 1.0 + 5 * (1.0 + 4.0))
    # two gradient slots: the write-backs run back to back after the first dW
    t = cf.ring_pass_time(5, 2, 0.1, backward=True, t_dx=1.0, t_dw=1.0, t_back=4.0, grad_slots=2)
    assert t == pytest.approx(0.1 + 1.0 + 1.0 + 5 * 4.0)


def test_paired_dx_by_hand():
    # N = 4, d = 2, copy 2, dX 1, dW 1, free write-back, two gradient slots.
    # Paired: tile 0 copy [0,2] dW [2,3]; tile 1 copy [2,4], dX of both [4,6]
    # frees both slots, dW [6,7]; tile 2 copy [6,8] dW [8,9]; tile 3 copy
    # [8,10], dX of both [10,12], dW [12,13]
    b = {"t_copy": 2.0, "backward": True, "t_dx": 1.0, "t_dw": 1.0, "t_back": 0.0}
    assert cf.ring_run(4, 2, [dict(b, pairs=True)], grad_slots=2) == [13.0]
    # unpaired: tile 0 dX [2,3] dW [3,4]; tile 1 copy [2,4] dX [4,5] dW [5,6];
    # tile 2 copy [4,6] (slot 0 free at 3) dX [6,7] dW [7,8]; tile 3 copy
    # [6,8] dX [8,9] dW [9,10]
    assert cf.ring_run(4, 2, [b], grad_slots=2) == [10.0]
    # compute-bound, the pairing costs nothing: one copy, then every product
    fast = dict(b, t_copy=0.5, pairs=True)
    assert cf.ring_run(4, 3, [fast], grad_slots=2) == [0.5 + 0.0 + 4 * 2.0]
    # an odd count leaves the last tile on its own
    assert cf.ring_run(3, 2, [dict(b, t_copy=0.5, pairs=True)], grad_slots=2) == [0.5 + 3 * 2.0]
    with pytest.raises(ValueError):
        cf.ring_run(4, 2, [dict(b, pairs=True)], grad_slots=0)


def test_paired_recompute_by_hand():
    # N = 4, d = 2, copy 2, recompute 1, dX 1, dW 1, free write-back, two
    # gradient slots, dX paired.  Recompute per tile: tile 0 copy [0,2]
    # recompute [2,3] dW [3,4]; tile 1 copy [2,4] recompute [4,5] dX [5,7]
    # dW [7,8]; tile 2 copy [7,9] (both slots freed at 7) recompute [9,10]
    # dW [10,11]; tile 3 copy [9,11] recompute [11,12] dX [12,14] dW [14,15].
    b = {"t_copy": 2.0, "backward": True, "t_re": 1.0, "t_dx": 1.0, "t_dw": 1.0, "t_back": 0.0,
         "pairs": True}
    assert cf.ring_run(4, 2, [b], grad_slots=2) == [15.0]
    # re_pairs: tile 0 dW [2,3]; tile 1 copy [2,4] recompute of both [4,6]
    # dX [6,8] dW [8,9]; tile 2 copy [8,10] dW [10,11]; tile 3 copy [10,12]
    # recompute [12,14] dX [14,16] dW [16,17]: link-bound, holding the slots
    # through the pair's recompute costs its time once per pair
    assert cf.ring_run(4, 2, [dict(b, re_pairs=True)], grad_slots=2) == [17.0]
    # compute-bound the order costs nothing in this model, which prices a
    # product by its FLOPs (the pair's gain is in rounds of workgroups)
    fast = dict(b, t_copy=0.5)
    assert cf.ring_run(4, 2, [fast], grad_slots=2) == [12.5]
    assert cf.ring_run(4, 2, [dict(fast, re_pairs=True)], grad_slots=2) == [12.5]
    # re_pairs without pairs changes nothing
    assert cf.ring_run(4, 2, [dict(b, pairs=False, re_pairs=True)], grad_slots=2) == \
        cf.ring_run(4, 2, [dict(b, pairs=False)], grad_slots=2)


def test_ring_bytes_reading():
    K, n = 1024, 512
    tile = K * n * 2
    assert cf.ring_bytes(K, n, 2, "f16", 0, False) == (0, 2 * tile)
    assert cf.ring_bytes(K, n, 2, "f16", 0, True) == (2, 4 * tile)
    assert cf.ring_bytes(K, n, 2, "f16", 3 * tile, True) == (1, 3 * tile)
    assert cf.ring_bytes(K, n, 2, "f16", 2 * tile, True) == (0, 2 * tile)
    assert cf.ring_bytes(K, n, 3, "f16", 2 * tile, True) is None
    # an fp32 gradient does not fit a 16-bit weight slot
    assert cf.ring_bytes(K, n, 2, "f16", 2 * tile, True, grad_f32=True) is None


def rates(widths, f):
    r = [f(n) for n in widths]
    return r, r, r


def test_flat_rates_fast_link_pick_the_finest_tiles():
    # every product at the same rate and copies faster than products: the pass
    # costs the first copy plus all products, so the smallest width wins, at
    # d = 2 (d = 1 overlaps nothing; d = 3 only costs more memory)
    T, K, M = 4096, 8192, 32768
    widths = [512, 1024, 2048, 4096, 8192]
    r = rates(widths, lambda n: 1e15)
    best, table = cf.choose_tiling(T, K, M, "bf16", 0, widths, *r, h2d=5e13, d2h=5e13, backward=1, max_d=3)
    assert (best["n"], best["d"]) == (512, 2)
    assert len(table) == 15
    fwd = [c for c in table if c["n"] == 512 and c["d"] == 2][0]
    assert fwd["t_fwd_s"] == pytest.approx(K * 512 * 2 / 5e13 + 2.0 * T * K * M / 1e15, rel=1e-12)


def test_slow_small_products_move_the_choice():
    # rate(n) = 1e15 * n / (n + 2048): small tiles lose throughput.  Every
    # tile's copy is shorter than its product (T * h2d > rate).  A forward on
    # its own costs t_copy(n) + 2TKM / rate(n) at d = 2; among back-to-back
    # steps the next pass's first copy runs under this pass's last product,
    # so a step costs 2TKM / rate(n) alone and the widest tile wins.
    T, K, M = 65536, 8192, 65536
    widths = [256, 512, 1024, 2048, 4096, 8192, 16384, 32768]
    rate = lambda n: 1e15 * n / (n + 2048)
    r = rates(widths, rate)
    h2d = 5e10
    best, table = cf.choose_tiling(T, K, M, "f16", 0, widths, *r, h2d=h2d, d2h=h2d, backward=0, max_d=2)
    assert best["n"] == 32768 and best["d"] == 2
    for c in table:
        n = c["n"]
        if c["d"] == 2:
            assert c["t_fwd_s"] == pytest.approx(K * n * 2 / h2d + 2.0 * T * K * M / rate(n), rel=1e-12)
            assert c["t_step_s"] == pytest.approx(2.0 * T * K * M / rate(n), rel=1e-12)
        else:
            assert c["t_step_s"] == pytest.approx(M // n * (K * n * 2 / h2d) + 2.0 * T * K * M / rate(n),
                                                  rel=1e-12)


def test_steady_steps_by_hand():
    # two forward passes of N = 2 tiles on d = 2 slots, copy 1, product 3:
    # pass 1 copies [0,1] [1,2], products [1,4] [4,7]; pass 2's first copy
    # waits for slot 0 (free at 4): [4,5], its second for slot 1 (free at 7):
    # [7,8]; products [7,10] [10,13]
    p = {"t_copy": 1.0, "t_fwd": 3.0}
    assert cf.ring_run(2, 2, [p, p]) == [7.0, 13.0]
    # compute-bound, link-bound and serial steady states
    assert cf.steady_step_time(5, 2, [p]) == 5 * 3.0
    assert cf.steady_step_time(5, 3, [{"t_copy": 4.0, "t_fwd": 1.0}]) == 5 * 4.0
    assert cf.steady_step_time(5, 1, [p]) == 5 * (1.0 + 3.0)
    # forward then backward (two gradient slots, free write-back): the step is
    # its products, back to back
    b = {"t_copy": 1.0, "backward": True, "t_dx": 2.0, "t_dw": 2.0, "t_back": 0.0}
    assert cf.steady_step_time(4, 2, [p, b], grad_slots=2) == 4 * 3.0 + 4 * 4.0


def test_budget_excludes_wide_tiles():
    T, K, M = 4096, 8192, 32768
    widths = [1024, 2048, 4096, 8192]
    r = rates(widths, lambda n: 1e15 * n / (n + 512))
    budget = 2 * K * 2048 * 2  # two weight slots of the 2048-wide tile
    best, table = cf.choose_tiling(T, K, M, "bf16", budget, widths, *r, h2d=5e10, d2h=5e10,
                                   backward=1, max_d=3)
    assert all(c["ring_bytes"] <= budget for c in table)
    # 4096-wide tiles fit only one slot; 8192-wide ones not even that
    assert {c["d"] for c in table if c["n"] == 4096} == {1}
    assert max(c["n"] for c in table) == 4096
    # the 2048-wide tiles fit d = 2 with the gradient formed in the weight slot
    assert [c["dw_slots"] for c in table if c["n"] == 2048 and c["d"] == 2] == [0]
    none, table = cf.choose_tiling(T, K, M, "bf16", 1000, widths, *r, h2d=5e10, d2h=5e10,
                                   backward=1, max_d=3)
    assert none is None and table == []


def test_link_bound_flat_rates():
    # copies slower than products: N copies back to back then the last
    # product, so again the finest tiles win (the last product is shortest)
    T, K, M = 256, 8192, 32768
    widths = [1024, 4096, 16384]
    r = rates(widths, lambda n: 1e15)
    best, table = cf.choose_tiling(T, K, M, "f16", 0, widths, *r, h2d=5e10, d2h=5e10, backward=0, max_d=2)
    assert (best["n"], best["d"]) == (1024, 2)
    c = [x for x in table if x["n"] == 1024 and x["d"] == 2][0]
    assert c["t_fwd_s"] == pytest.approx(K * M * 2 / 5e10 + 2.0 * T * K * 1024 / 1e15, rel=1e-12)
