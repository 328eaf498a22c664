"""Host threading of the library on the CPU: the file tier's read-ahead under
a consumer that stages tiles in and out of the traced order, and the host
optimizer's engine under two optimizers made and destroyed in rounds.  Each
program in tests/native compiles the library source it tests with host
stand-ins for the HIP calls it makes."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def build_and_run(tmp_path, name, *args):
    exe = str(tmp_path / name)
    build = subprocess.run(["g++", "-O1", "-std=c++17", "-pthread", "-mavx2", "-mf16c", "-I/opt/rocm/include",
                            "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "native", name + ".cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe, *args], capture_output=True, text=True, timeout=240)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "bad 0" in run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tier_read_ahead_stress(tmp_path):
    build_and_run(tmp_path, "tier_stress", str(tmp_path))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_adam_engine_stress(tmp_path):
    build_and_run(tmp_path, "adam_engine_stress")
