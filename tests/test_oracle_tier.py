"""The file tier's cache policy: the oracle's rewrite of it pinned to a
hand-worked trace, to Belady's offline optimum (no policy reads less) and to
the case where every tile fits; the library's simulation of the same policy
(zi_tier_simulate_reads) against the oracle.  CPU only."""
import random

import pytest

from oracle import closed_forms as cf


def test_hand_worked_trace():
    # trace A B A C with two buffers.  Step 0: A, B read; A held; C evicts B
    # (B is next wanted after A).  Step 1: A held; B evicts C; A held; C
    # evicts B.  3 then 2 reads, as the offline optimum.
    tr = ["A", "B", "A", "C"]
    assert cf.tier_policy_reads(tr, 2, 2) == [3, 2]
    assert cf.belady_reads(tr, 2, 2) == [3, 2]


def test_every_tile_fits():
    tr = [("w1", t) for t in range(6)] * 3 + [("w2", t) for t in range(6)] * 2
    for buffers in (12, 13, 20):
        reads = cf.tier_policy_reads(tr, buffers, 4)
        assert reads == [12, 0, 0, 0]


def test_never_below_the_optimum():
    rng = random.Random(5)
    for _ in range(40):
        items = rng.randint(2, 9)
        tr = [rng.randrange(items) for _ in range(rng.randint(3, 25))]
        buffers = rng.randint(2, 8)
        steps = rng.randint(1, 4)
        ours, best = cf.tier_policy_reads(tr, buffers, steps), cf.belady_reads(tr, buffers, steps)
        assert sum(ours) >= sum(best), (tr, buffers)
        assert sum(ours) <= steps * len(tr)


def test_block_trace_reads():
    # the feed-forward block's step: W1's 16 tiles three times, W2's twice
    tr = [("w1", t) for t in range(16)] + [("w2", t) for t in range(16)] + [("w1", t) for t in range(16)] + \
        [("w2", t) for t in range(16)] + [("w1", t) for t in range(16)]
    best = [cf.belady_reads(tr, c, 4)[3] for c in (8, 16, 24, 32)]
    assert best[-1] == 0 and best == sorted(best, reverse=True)
    ours = [cf.tier_policy_reads(tr, c, 4)[3] for c in (8, 16, 24, 32, 40)]
    assert ours[-1] == 0
    assert all(o >= b for o, b in zip(ours, best))


def test_one_ahead_is_at_least_as_good_as_the_optimum_with_one_slot_less():
    # with the reads one request ahead, one buffer waits for the next request
    # and the others cache: never more reads than the optimum with one slot less
    rng = random.Random(7)
    for _ in range(40):
        items = rng.randint(2, 9)
        tr = [rng.randrange(items) for _ in range(rng.randint(3, 25))]
        buffers = rng.randint(2, 8)
        assert sum(cf.tier_policy_reads(tr, buffers, 3, window=1)) <= sum(cf.belady_reads(tr, buffers - 1, 3))


@pytest.mark.parametrize("seed", range(25))
def test_library_simulation_matches_the_oracle(seed):
    from offload_memory_centric_amd import zi
    rng = random.Random(100 + seed)
    items = rng.randint(2, 12)
    tr = [rng.randrange(items) for _ in range(rng.randint(1, 40))]
    buffers = rng.randint(2, 10)
    window = rng.randint(1, buffers)
    steps = rng.randint(1, 5)
    assert zi.zi_tier_simulate_reads(tr, buffers, steps) == cf.tier_policy_reads(tr, buffers, steps)
    assert zi.zi_tier_simulate_reads(tr, buffers, steps, window) == cf.tier_policy_reads(tr, buffers, steps, window)


def test_library_simulation_errors():
    from offload_memory_centric_amd import zi
    for args in (([], 2, 1), ([1, 2], 1, 1), ([1, 2], 2, 0), ([1, 2], 2, 1, 3)):
        with pytest.raises(zi.ZiError) as e:
            zi.zi_tier_simulate_reads(*args)
        assert e.value.status == zi.ZI_ERR_ARG
