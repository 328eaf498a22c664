"""The MFMA wait-state check that the build runs on the kernels' assembly.

The GEMM kernels issue their MFMAs (and the loads of an accumulating
product's C) as inline assembly, which the compiler neither pads with wait
states nor waits for.  These tests plant each kind of mistake in a small
hand-written listing and require the check to report it, and require a clean
listing to pass; the last one checks the assembly the build kept, if any.
"""
import os

import pytest

from offload_memory_centric_amd import asm_check, build

HEAD = "_ZN2zi6kernelEv:\n"
TAIL = "\ts_endpgm\n"


def findings(body: str):
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), "asm_check_case_%d.s" % os.getpid())
    with open(path, "w") as f:
        f.write(HEAD + body + TAIL)
    try:
        res = asm_check.check_file(path)
    finally:
        os.remove(path)
    assert list(res) == ["_ZN2zi6kernelEv"]
    return res["_ZN2zi6kernelEv"]


MFMA = "\tv_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]\n"
DRAIN = "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n"


def test_clean_sequence_passes():
    body = ("\tv_accvgpr_write_b32 a0, 0\n\ts_nop 1\n" + MFMA + MFMA + DRAIN +
            "\tv_accvgpr_read_b32 v8, a0\n")
    assert findings(body) == []


def test_result_read_too_early():
    assert findings(MFMA + "\ts_nop 3\n\tv_accvgpr_read_b32 v8, a2\n")


def test_result_spilled_too_early():
    assert findings(MFMA + "\tscratch_store_dwordx4 off, a[0:3], off\n")


def test_accumulator_written_right_before_mfma():
    assert findings("\tv_accvgpr_write_b32 a1, 0\n" + MFMA)
    assert findings("\tv_accvgpr_mov_b32 a3, a9\n\ts_nop 0\n" + MFMA)
    assert findings("\tv_accvgpr_write_b32 a1, 0\n\ts_nop 1\n" + MFMA) == []


def test_operand_from_mfma_in_flight():
    body = "\tv_mfma_f32_16x16x32_f16 a[8:11], v[0:3], v[4:7], a[8:11]\n" \
           "\tv_mfma_f32_16x16x32_f16 a[0:3], a[8:11], v[4:7], a[0:3]\n"
    assert findings(body)


def test_partial_accumulator_overlap():
    body = "\tv_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]\n" \
           "\tv_mfma_f32_16x16x32_f16 a[2:5], v[0:3], v[4:7], a[2:5]\n"
    assert findings(body)


def test_back_edge_is_followed():
    # the read at the loop head follows the MFMA at its end on the next pass
    body = (".LBB0_1:\n\tv_accvgpr_read_b32 v8, a1\n" + DRAIN + DRAIN + MFMA +
            "\ts_cbranch_scc1 .LBB0_1\n" + DRAIN)
    assert findings(body)


def test_load_into_accumulators_needs_a_wait():
    load = "\tbuffer_load_dwordx4 a[0:3], v9, s[0:3], 0 offen\n"
    copy = "\tbuffer_load_dwordx4 v10, s[4:7], 0 offen lds\n"
    assert findings(load + MFMA)
    assert findings(load + copy + "\ts_waitcnt vmcnt(1)\n" + MFMA) == []
    assert findings(load + copy + "\ts_waitcnt vmcnt(2)\n" + MFMA)
    assert findings(load + "\tv_accvgpr_mov_b32 a4, a0\n")


def test_m0_only_for_lds_copies():
    copy = "\ts_mov_b32 m0, s4\n\tbuffer_load_dwordx4 v10, s[4:7], 0 offen lds\n"
    assert findings(copy) == []
    assert findings("\ts_mov_b32 m0, s4\n\ts_nop 0\n\tbuffer_load_dwordx4 v10, s[4:7], 0 offen lds\n")
    assert findings(copy + "\ts_add_u32 s5, m0, 4\n")


def test_built_kernels_pass():
    path = build.device_asm()
    if not os.path.exists(path):
        pytest.skip("library not built")
    res = asm_check.check_file(path, "gemm_kernel")
    assert res, "no GEMM kernels in the kept assembly"
    assert {k: v for k, v in res.items() if v} == {}
