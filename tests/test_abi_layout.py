"""The binding's ctypes structures have the C header's layout: a small C
program built with gcc prints the size and every field offset of each struct
in include/zi.h, and the ctypes mirror must agree field by field."""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = ["zi_problem", "zi_plan_info", "zi_prediction", "zi_rate_curve", "zi_choice", "zi_kernel_stats",
           "zi_stats", "zi_timed_rec", "zi_adam_hparams", "zi_adam_stats", "zi_source_stats", "zi_tier_stats"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_ctypes_structs_match_the_header(tmp_path):
    from offload_memory_centric_amd import zi
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "zi.h"', "int main(void) {"]
    for name in STRUCTS:
        cls = getattr(zi, name)
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (name, name))
        for field, _ in cls._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (name, field, name, field))
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = str(tmp_path / "layout")
    b = subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", exe],
                       capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            a, f, v = line.split()
            got[(a, f)] = int(v)
    for name in STRUCTS:
        cls = getattr(zi, name)
        assert ctypes.sizeof(cls) == got[(name, "size")], name
        for field, _ in cls._fields_:
            assert getattr(cls, field).offset == got[(name, field)], (name, field)
