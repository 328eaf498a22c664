"""bench.py's command-line contract on the CPU: a request for more than one
GPU ends with a message and a non-zero status before anything touches a
device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_trace_labels_of_the_gemm_instances():
    # rocprofv3 reports the mangled kernel names; the summaries label them by
    # template arguments and workgroup count (grid in threads / 256)
    sys.path.insert(0, ROOT)
    import bench

    pre = "_ZN2zi12_GLOBAL__N_111gemm_kernelI"
    suf = "EvNS_8GemmArgsEii"
    assert bench.kernel_label(pre + "DF16_Lb0ELb0ELi2ELb1ELi8ELi8ELb0EE" + suf, 3200 * 256, 256) == \
        "gemm<f16,rc,rc,gelu,8x8> x3200"
    assert bench.kernel_label(pre + "DF16_Lb1ELb0ELi3ELb1ELi8ELi8ELb1EE" + suf, 256 * 256, 256) == \
        "gemm<f16,rs,rc,acc,8x8,persistent> x256"
    assert bench.kernel_label(pre + "DF16bLb1ELb1ELi1ELb0ELi6ELi10ELb0EE" + suf, 2670 * 256, 256) == \
        "gemm<bf16,rs,rs,f32,6x10,ragged> x2670"
    # names from before the persistent flag existed
    assert bench.kernel_label(pre + "DF16_Lb0ELb0ELi0ELb1ELi10ELi6EE" + suf, 855 * 256, 256) == \
        "gemm<f16,rc,rc,lp,10x6> x855"
    assert bench.kernel_label("void at::native::foo<float>(int)", 1024, 256) == "at::native::foo<float> x4"
    assert bench.kernel_label("_ZN2zi12_GLOBAL__N_115gelu_bwd_kernelIDF16_Lb0EEEvPKfPKtPvl", 256 * 1024, 1024) == \
        "gelu_bwd x256"
    assert bench.kernel_label("_ZN2zi12_GLOBAL__N_122gelu_grad_table_kernelIDF16bEEvv", 256 * 256, 256) == \
        "gelu_grad_table x256"
    assert bench.kernel_label("_ZN2zi12_GLOBAL__N_117gelu_table_kernelIDF16_EEvv", 256 * 256, 256) == \
        "gelu_table x256"


def test_split_labels_by_dispatch_order():
    # launches of one kernel and grid told apart by their order: runs of 2
    # and 1 repeating, keyed by dispatch id (not by list position)
    sys.path.insert(0, ROOT)
    import bench

    labels = ["k", "other", "k", "k", "k", "k", "k"]
    keys = [5, 1, 2, 9, 7, 3, 11]  # dispatch ids: k's order is 2, 3, 5, 7, 9, 11
    out = bench.split_labels(keys, labels, {"k": [2, 1]})
    by_key = dict(zip(keys, out))
    assert by_key[1] == "other"
    assert [by_key[k] for k in (2, 3, 5, 7, 9, 11)] == ["k #0", "k #0", "k #1", "k #0", "k #0", "k #1"]
    assert bench.split_labels(keys, labels, {}) == labels


def test_comparison_switches_parse(monkeypatch):
    # the switches that select the other form of a kernel for an alternated
    # comparison parse, and default to the built form
    sys.path.insert(0, ROOT)
    import bench

    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert not a.no_gelu_split and not a.dx_per_tile
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-gelu-split", "--dx-per-tile"])
    a = bench.parse()
    assert a.no_gelu_split and a.dx_per_tile
