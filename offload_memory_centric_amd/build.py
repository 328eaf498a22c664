"""Build libzi.so (the C-ABI library) in-tree for gfx950 with hipcc.

Run ``python -m offload_memory_centric_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzi.so")
OBJDIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
SOURCES = ["zi_kernels.hip", "zi_api.cpp", "zi_plan.cpp", "zi_adam.cpp", "zi_source.cpp", "zi_noalloc.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
# Packed fp32 VALU forms are kept out of every device code object.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def device_asm(src: str = "zi_kernels.hip") -> str:
    """Path of the gfx950 assembly that the build keeps for a HIP source."""
    stem = os.path.splitext(os.path.basename(src))[0]
    return os.path.join(OBJDIR, "%s-hip-amdgcn-amd-amdhsa-%s.s" % (stem, ARCH))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    # HIP sources keep their intermediate files next to the object, so that
    # the device assembly that went into the object can be checked.
    temps = ["-save-temps=obj"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + COMMON + DEVICE + temps + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    if temps:
        keep = device_asm(src)
        stem = os.path.splitext(os.path.basename(src))[0]
        for f in os.listdir(OBJDIR):
            if f.startswith(stem + "-") or f.startswith(os.path.basename(src) + "-"):
                if os.path.join(OBJDIR, f) != keep:
                    os.remove(os.path.join(OBJDIR, f))
    return obj


def check_device_asm(src: str = "zi_kernels.hip") -> None:
    """Fail unless the kernels' matrix-core instructions keep their required
    wait states (the MFMAs are inline assembly, which the compiler does not
    pad)."""
    from . import asm_check
    path = device_asm(src)
    res = asm_check.check_file(path)
    bad = {k: v for k, v in res.items() if v}
    if not res:
        raise RuntimeError("no kernels found in %s" % path)
    if bad:
        lines = ["%s: %s" % (k, v[0]) for k, v in bad.items()]
        raise RuntimeError("MFMA wait-state check failed in %d kernels:\n%s" % (len(bad), "\n".join(lines)))


def build(verbose: bool = False) -> str:
    """Compile every source and link libzi.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    check_device_asm()
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
