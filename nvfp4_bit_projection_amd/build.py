"""Build step of the HIP library (hipcc, gfx950 only).

``build_library()`` compiles ``csrc/*.hip`` (device and host code) and
``csrc/*.cpp`` (host-only code) into ``libflint_moe.so`` next to this file.  All device code is built with packed FP32 instructions disabled
(``-target-feature -packed-fp32-ops``), so the compiler emits only scalar
FP32 FMAs.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflint_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) + glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build_library(out: str = LIB_PATH) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *COMMON_FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"), *sources(), "-o", tmp]
    subprocess.run(cmd, check=True, stderr=subprocess.PIPE)
    os.replace(tmp, out)
    return out
