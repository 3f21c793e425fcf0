"""The library from a plain C client (CPU only): tests/c/abi_probe.c is built
with gcc against include/mla_post.h alone (C99, warnings as errors) and
linked to the built library. The struct layout C sees must equal the Python
binding's, and validation must give the status codes the header documents.
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest

import mla_split_kv_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "c", "abi_probe.c")
ROCM_LIB = "/opt/rocm/lib"

OK, EINVAL, ESTRIDE, EALIGN, EUNSUP = 0, -1, -2, -3, -5

EXPECTED = {
    "valid": OK,
    "null_struct": EINVAL,
    "null_o": EINVAL,
    "null_lse_n4": EINVAL,  # lse may be NULL only when n == 1
    "null_lse_n1": OK,
    "odd_o_stride": ESTRIDE,  # o strides must be multiples of 8 elements
    "misaligned_core": EALIGN,  # core must be 16-byte aligned
    "n_too_large": EUNSUP,  # n above MLA_POST_NMAX
    "negative_S": EINVAL,
    "q_not_dividing_S": EINVAL,
    "v1_ignores_q": OK,  # a version-1 struct_size: q is not read
    "struct_too_small": EINVAL,
    "launch_odd_o_stride": ESTRIDE,  # mla_post validates before anything else
    "launch_empty": OK,  # S == 0 is a no-op
    "quantize_bad_cols": EUNSUP,  # cols not a multiple of 32
}


@pytest.fixture(scope="module")
def probe_output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    m.load()  # the library must be built
    libdir = os.path.dirname(m.LIB_PATH)
    exe = str(tmp_path_factory.mktemp("cabi") / "abi_probe")
    cmd = [
        "gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
        "-I", os.path.join(ROOT, "include"), PROBE, "-o", exe,
        "-L", libdir, "-lmla_post", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath-link,{ROCM_LIB}",
    ]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = ROCM_LIB + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=60).stdout
    sizes, offsets, statuses = {}, {}, {}
    for line in out.splitlines():
        parts = line.split()
        if parts[0] == "offset":
            offsets[parts[1]] = int(parts[2])
        elif parts[0] == "plan_offset":
            offsets["plan." + parts[1]] = int(parts[2])
        elif parts[0] in ("plan_large", "plan_tiny") and parts[1].lstrip("-").isdigit():
            sizes[parts[0]] = [int(x) for x in parts[1:]]
        elif parts[0] == "status":
            statuses[parts[1]] = int(parts[2])
        elif parts[0] in ("sizeof", "v1_size", "header_version", "library_version", "plan_sizeof"):
            sizes[parts[0]] = int(parts[1])
    return sizes, offsets, statuses


def test_struct_layout_matches_binding(probe_output):
    sizes, offsets, _ = probe_output
    assert sizes["sizeof"] == ctypes.sizeof(m.MlaPostArgs) == 224
    assert sizes["v1_size"] == m.ARGS_V1_SIZE == offsets["q"]
    args_offsets = {k: v for k, v in offsets.items() if not k.startswith("plan.")}
    assert args_offsets == {name: getattr(m.MlaPostArgs, name).offset for name, _ in m.MlaPostArgs._fields_}


def test_plan_from_c(probe_output):
    """mla_post_plan as C sees it matches the binding's struct, and the plan
    query gives from C what it gives from Python (256 CUs)."""
    sizes, offsets, statuses = probe_output
    assert sizes["plan_sizeof"] == ctypes.sizeof(m.MlaPostPlan) == 40
    plan_offsets = {k[5:]: v for k, v in offsets.items() if k.startswith("plan.")}
    assert plan_offsets == {name: getattr(m.MlaPostPlan, name).offset for name, _ in m.MlaPostPlan._fields_}
    assert statuses["plan_large"] == statuses["plan_tiny"] == OK
    assert sizes["plan_large"] == [2, 768, 4, 256]  # persistent, 768 workgroups, 4 full tiles each
    assert sizes["plan_tiny"] == [1, 8, 2, 12]      # one-tile, 8-token tiles, 2 rows, 12 workgroups
    assert statuses["plan_bad_stride"] == ESTRIDE and statuses["plan_null_out"] == EINVAL


def test_versions_agree(probe_output):
    sizes, _, _ = probe_output
    assert sizes["header_version"] == sizes["library_version"] == 5


def test_status_codes_from_c(probe_output):
    _, _, statuses = probe_output
    assert {k: v for k, v in statuses.items() if not k.startswith("plan_")} == EXPECTED
