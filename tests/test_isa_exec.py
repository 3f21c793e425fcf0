"""The MFMAs of every kernel run with the whole wave active (CPU only).

A scaled FP4 MFMA reads its operands from all 64 lanes; issued under a
narrowed exec mask (inside a lane-dependent branch, such as the per-lane
store of a ragged tile) it would compute with stale operands. The kernels
keep every MFMA ahead of lane-dependent control flow by construction (the
result goes to an unconditional LDS store); this test compiles the device
code to gfx950 assembly and checks the built code: no v_mfma lies inside a
region where exec has been narrowed (s_and_saveexec / s_and exec ... up to
the s_or exec that restores it; the compiler emits structured regions, so a
linear scan tracks their nesting). The same scan must find narrowed regions
around some stores, which shows that it sees them at all.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mla_split_kv_amd", "csrc", "mla_post.hip")

NARROW = re.compile(r"s_(and|andn2|or|xor)_saveexec_b64|s_(and|andn2|xor)_b64\s+exec,")
RESTORE = re.compile(r"s_or_b64\s+exec,\s*exec")


def exec_depths(asm: str):
    """(function, mnemonic, depth) for every MFMA and vector store."""
    fn, depth, out = None, 0, []
    for line in asm.splitlines():
        l = line.strip()
        m = re.match(r"^(_Z[_A-Za-z0-9]+):", l)
        if m:
            fn, depth = m.group(1), 0
            continue
        if NARROW.match(l):
            depth += 1
        elif RESTORE.match(l):
            depth = max(0, depth - 1)
        if l.startswith("v_mfma") or re.match(r"(global|buffer)_store", l):
            out.append((fn, l.split()[0], depth))
    return out


def device_asm(src: str, tmp_path) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out), src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


@pytest.mark.slow
def test_mfma_under_full_exec(tmp_path):
    rows = exec_depths(device_asm(SRC, tmp_path))
    mfma = [x for x in rows if x[1].startswith("v_mfma")]
    assert len(mfma) > 0, "no MFMA found in the device code"
    masked = [x for x in mfma if x[2] > 0]
    assert not masked, f"MFMAs under a narrowed exec mask: {masked[:5]}"
    assert any(d > 0 for _, m, d in rows if "store" in m), "the scan found no narrowed region at all"
