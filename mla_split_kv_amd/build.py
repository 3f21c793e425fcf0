"""Build libmla_post.so in-tree with hipcc for gfx950, and the C test client.

    python -m mla_split_kv_amd.build

Compiles every time it is called (the C-ABI library, its kernels and host code
from csrc/mla_post.hip, oproj.hip, decode.hip and measure.hip). Packed-FP32 instructions are disabled for the device
code; hipcc's host pass warns that it does not know that feature, harmlessly.
build_c_client compiles tests/c/c_client.c, a plain C program that calls the
library through the HIP runtime's C API, with gcc against include/ alone.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("mla_post.hip", "oproj.hip", "decode.hip", "measure.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_post.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c", "c_client")


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        "-I",
        INC,
        "-o",
        tmp,
    ] + SRCS
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_c_client() -> str:
    """gcc, C99, warnings as errors; linked to the in-tree library by a
    path relative to the executable, so the tree can move."""
    gcc = shutil.which("gcc")
    if gcc is None:
        raise RuntimeError("gcc not found")
    tmp = C_CLIENT + ".tmp"
    cmd = [
        gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", INC,
        C_CLIENT_SRC, "-o", tmp,
        "-L", PKG, "-lmla_post", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
        "-Wl,-rpath,$ORIGIN/../../mla_split_kv_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
    ]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(tmp, C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client())
