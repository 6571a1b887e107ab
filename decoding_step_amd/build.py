"""Build ``libdlm.so`` (the HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "dlm.hip")]
DEPS = SOURCES + [os.path.join(HERE, "csrc", "dlm_device.hpp"), os.path.join(ROOT, "include", "dlm.h")]
LIB = os.path.join(HERE, "libdlm.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def command(out: str = LIB) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # no packed-fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # device code sees no NaNs (every empty statistic is guarded by a select), so minimum and
        # maximum need no signalling-NaN quieting: IEEE mode off in the kernels
        "-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, *SOURCES,
    ]


def build(verbose: bool = False) -> str:
    """Compile unconditionally; returns the library path."""
    tmp = LIB + ".tmp"
    res = subprocess.run(command(tmp), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
