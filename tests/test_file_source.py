"""The file source's reads on the CPU (zi_file_source_read: no GPU involved):
every tile's bytes as the file holds them, at any offset and thread count,
and the error paths."""
import os

import numpy as np
import pytest

from offload_memory_centric_amd import zi


def plan(T=16, K=512, M=2048, N=4, dtype="f16"):
    prob = zi.zi_problem(T=T, K=K, M=M, N=N, d=2, dtype=zi.DTYPE_CODES[dtype], flags=0,
                         device_budget_bytes=0, W_host=None, dW_host=None)
    h, info = zi.zi_plan_tiles(prob)
    return h, info


def aligned(nbytes, align=4096):
    raw = np.empty(nbytes + align, np.uint8)
    at = (-raw.ctypes.data) % align
    return raw[at:at + nbytes]


@pytest.fixture
def weight_file(tmp_path):
    def make(nbytes, offset=0, seed=0):
        data = np.frombuffer(np.random.default_rng(seed).bytes(offset + nbytes), np.uint8)
        path = str(tmp_path / ("w_%d_%d.bin" % (offset, seed)))
        data.tofile(path)
        return path, data
    return make


@pytest.mark.parametrize("offset", [0, 4096, 100])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_tiles_read_back(weight_file, offset, threads):
    h, info = plan(K=1024, M=8192, N=4)  # 4 MiB tiles: several 8 MiB-or-less pieces per thread count
    try:
        path, data = weight_file(info.tile_bytes * 4, offset)
        src = zi.zi_file_source_create(h, path, offset, 2, threads)
        try:
            for t in range(4):
                dst = aligned(info.tile_bytes)
                zi.zi_file_source_read(src, t, dst)
                lo = offset + t * info.tile_bytes
                assert np.array_equal(dst, data[lo:lo + info.tile_bytes]), t
            st = zi.zi_file_source_stats_get(src)
            assert st["tiles_read"] == 0  # the synchronous reads are not read-ahead
            if offset % 4096:
                assert st["direct"] == 0  # an unaligned offset is read through the page cache
        finally:
            zi.zi_file_source_destroy(src)
    finally:
        zi.zi_plan_destroy(h)


def test_big_tile_split_over_threads(weight_file):
    # a 20 MiB tile: two pieces (16 and 4 MiB) dealt over the threads
    h, info = plan(K=2560, M=8192, N=2)
    try:
        assert info.tile_bytes == 2560 * 4096 * 2
        path, data = weight_file(info.tile_bytes * 2, 0, seed=3)
        src = zi.zi_file_source_create(h, path, 0, 3, 4)
        try:
            dst = aligned(info.tile_bytes)
            zi.zi_file_source_read(src, 1, dst)
            assert np.array_equal(dst, data[info.tile_bytes:])
        finally:
            zi.zi_file_source_destroy(src)
    finally:
        zi.zi_plan_destroy(h)


def test_errors(weight_file, tmp_path):
    h, info = plan()
    try:
        path, _ = weight_file(info.tile_bytes * 4 - 1)  # one byte short
        with pytest.raises(zi.ZiError) as e:
            zi.zi_file_source_create(h, path, 0, 2, 2)
        assert e.value.status == zi.ZI_ERR_IO
        with pytest.raises(zi.ZiError) as e:
            zi.zi_file_source_create(h, str(tmp_path / "missing.bin"), 0, 2, 2)
        assert e.value.status == zi.ZI_ERR_IO
        path, _ = weight_file(info.tile_bytes * 4, seed=1)
        for staging, threads in ((1, 2), (2, 0)):
            with pytest.raises(zi.ZiError) as e:
                zi.zi_file_source_create(h, path, 0, staging, threads)
            assert e.value.status == zi.ZI_ERR_ARG
        src = zi.zi_file_source_create(h, path, 0, 2, 2)
        try:
            with pytest.raises(zi.ZiError) as e:
                zi.zi_file_source_read(src, 4, aligned(info.tile_bytes))
            assert e.value.status == zi.ZI_ERR_ARG
            if zi.zi_file_source_stats_get(src)["direct"]:
                with pytest.raises(zi.ZiError) as e:
                    zi.zi_file_source_read(src, 0, aligned(info.tile_bytes + 1)[1:])
                assert e.value.status == zi.ZI_ERR_ALIGN
            # a file that shrinks after the source was made fails the read, not the process
            os.truncate(path, info.tile_bytes * 2)
            with pytest.raises(zi.ZiError) as e:
                zi.zi_file_source_read(src, 3, aligned(info.tile_bytes))
            assert e.value.status == zi.ZI_ERR_IO
        finally:
            zi.zi_file_source_destroy(src)
    finally:
        zi.zi_plan_destroy(h)


def test_tier_bookkeeping_without_a_gpu(weight_file):
    h, info = plan()
    try:
        p1, _ = weight_file(info.tile_bytes * 4, seed=5)
        p2, _ = weight_file(info.tile_bytes * 4, seed=6)
        with pytest.raises(zi.ZiError) as e:
            zi.zi_tier_create(1, 4)
        assert e.value.status == zi.ZI_ERR_ARG
        tier = zi.zi_tier_create(3, 4)
        s1 = zi.zi_file_source_create(h, p1, 0, 2, 2)
        s2 = zi.zi_file_source_create(h, p2, 0, 2, 2)
        zi.zi_tier_add(tier, s1)
        zi.zi_tier_add(tier, s2)
        with pytest.raises(zi.ZiError) as e:  # a source has one tier
            zi.zi_tier_add(tier, s1)
        assert e.value.status == zi.ZI_ERR_STATE
        with pytest.raises(zi.ZiError) as e:  # the tier goes first
            zi.zi_file_source_destroy(s1)
        assert e.value.status == zi.ZI_ERR_STATE
        st = zi.zi_tier_stats_get(tier)
        assert st["trace_len"] == 0 and st["steps"] == 0 and st["tiles_read"] == 0
        zi.zi_tier_step(tier)
        assert zi.zi_tier_stats_get(tier)["steps"] == 1
        # synchronous reads go straight to the file, tier or not
        dst = aligned(info.tile_bytes)
        zi.zi_file_source_read(s2, 2, dst)
        zi.zi_tier_destroy(tier)
        zi.zi_file_source_destroy(s1)
        zi.zi_file_source_destroy(s2)
    finally:
        zi.zi_plan_destroy(h)
