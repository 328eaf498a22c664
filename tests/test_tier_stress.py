"""The file tier's read-ahead under a consumer that stages tiles in and out
of the traced order, on the CPU (tests/native/tier_stress.cpp compiles
zi_source.cpp with host stand-ins for its HIP calls)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tier_read_ahead_stress(tmp_path):
    exe = str(tmp_path / "tier_stress")
    build = subprocess.run(["g++", "-O1", "-std=c++17", "-pthread", "-I/opt/rocm/include",
                            "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "native", "tier_stress.cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=240)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "bad 0" in run.stdout
