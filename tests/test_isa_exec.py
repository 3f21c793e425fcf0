"""The MFMAs of every kernel run with the whole wave active (CPU only).

A scaled FP4 MFMA reads its operands from all 64 lanes; issued under a
narrowed exec mask (inside a lane-dependent branch, such as the per-lane
store of a ragged tile) it would compute with stale operands. The kernels
keep every MFMA ahead of lane-dependent control flow by construction (the
result goes to an unconditional LDS store); this test compiles the device
code to gfx950 assembly and checks the built code: no v_mfma lies inside a
region where exec may have been narrowed (s_and_saveexec / s_and exec ...
up to the s_or exec that restores it, tracked over the control-flow graph of
each kernel). The same scan must find narrowed regions around some stores,
which shows that it sees them at all.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_split_kv_amd", "csrc")
# the sources with MFMAs: their own, or the shared helpers' (post_common.h)
SRCS = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
              if f.endswith(".hip") and any(k in open(os.path.join(CSRC, f)).read()
                                            for k in ("__builtin_amdgcn_mfma", '#include "post_common.h"')))

NARROW_SAVE = re.compile(r"s_(and|andn2|or|xor)_saveexec_b64\s+(s\[\d+:\d+\]|vcc)")
NARROW_OP = re.compile(r"s_(and|andn2|xor)_b64\s+exec,\s*exec,\s*(s\[\d+:\d+\]|vcc)")
RESTORE = re.compile(r"s_or_b64\s+exec,\s*exec,\s*(s\[\d+:\d+\])")
# an if/else: after the then-branch's saveexec into sY, s_xor sX, exec, sY
# holds the else lanes; s_andn2_saveexec sX, sX switches exec to them (the
# same depth), and s_or exec, exec, sX restores the exec of before the if
ELSE_MASK = re.compile(r"s_xor_b64\s+(s\[\d+:\d+\]),\s*exec,\s*(s\[\d+:\d+\])")
ELSE_SWITCH = re.compile(r"s_andn2_saveexec_b64\s+(s\[\d+:\d+\]),\s*(s\[\d+:\d+\])")
# the same narrowing written out: s_mov sX, exec saves exec, s_and sY, sX, cond
# forms the mask, s_mov exec, sY narrows, s_or exec, exec, sX restores
SAVE_MOV = re.compile(r"s_mov_b64\s+(s\[\d+:\d+\]),\s*exec\b")
SET_MOV = re.compile(r"s_mov_b64\s+exec,\s*(s\[\d+:\d+\])")


def functions(asm: str) -> dict:
    """Kernel name -> its instruction and label lines."""
    fn, out = None, {}
    for line in asm.splitlines():
        l = line.strip()
        m = re.match(r"^(_Z[_A-Za-z0-9]+):", l)
        if m:
            fn = m.group(1)
            out[fn] = []
            continue
        if fn is None:
            continue
        if l.startswith(".Lfunc_end"):
            fn = None
            continue
        out[fn].append(l)
    return out


def basic_blocks(lines):
    """Basic blocks (label, instructions, successors) in layout order."""
    bl, cur = [], {"label": None, "ins": []}
    for l in lines:
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            bl.append(cur)
            cur = {"label": m.group(1), "ins": []}
            continue
        if not l or l.startswith(";") or l.startswith("."):
            continue
        cur["ins"].append(l)
        if re.match(r"s_(branch|cbranch_\w+|endpgm|setpc_b64)\b", l):
            bl.append(cur)
            cur = {"label": None, "ins": []}
    bl.append(cur)
    bl = [b for b in bl if b["ins"] or b["label"]]
    idx = {b["label"]: i for i, b in enumerate(bl) if b["label"]}
    for i, b in enumerate(bl):
        last = b["ins"][-1] if b["ins"] else ""
        succ = []
        m = re.match(r"s_branch\s+(\.LBB\d+_\d+)", last)
        if m:
            succ = [idx[m.group(1)]]
        elif not re.match(r"s_(endpgm|setpc_b64)", last):
            m = re.match(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", last)
            if m:
                succ.append(idx[m.group(1)])
            if i + 1 < len(bl):
                succ.append(i + 1)
        b["succ"] = succ
    return bl


def depth(st: tuple) -> int:
    """Exec narrowings in force (entries starting with "=" only record the
    latest copy of exec, see step)."""
    return sum(1 for e in st if not e.startswith("="))


def step(st: tuple, l: str) -> tuple:
    """The stack of exec narrowings after instruction l: a saveexec or an
    and/andn2/xor of exec pushes the register it uses; the s_or of exec with a
    saved register pops back to that register's entry. An entry holds the
    registers that restore it ("sY|sX" once an if/else's else mask sX is
    formed from sY); switching to the else branch keeps the depth. The
    written-out form: s_mov sX, exec records "=sX"; s_mov exec, sY then
    pushes sX (or "?" with no copy recorded, which the next s_or of exec with
    a register not on the stack pops)."""
    m = SAVE_MOV.match(l)
    if m:
        return tuple(e for e in st if not e.startswith("=")) + ("=" + m.group(1),)
    m = SET_MOV.match(l)
    if m:
        saved = [e[1:] for e in st if e.startswith("=")]
        rest = tuple(e for e in st if not e.startswith("="))
        return rest + ((saved[-1] if saved else "?"),)
    m = ELSE_MASK.match(l)
    if m and st and m.group(2) in st[-1].split("|"):
        return st[:-1] + (st[-1] + "|" + m.group(1),)
    m = ELSE_SWITCH.match(l)
    if m and st and m.group(1) == m.group(2) and m.group(1) in st[-1].split("|"):
        return st
    m = NARROW_SAVE.match(l) or NARROW_OP.match(l)
    if m:
        return st + (m.group(2),)
    m = RESTORE.match(l)
    if m:
        hits = [j for j, r in enumerate(st) if m.group(1) in r.split("|")]
        if not hits:
            hits = [j for j, r in enumerate(st) if r == "?"]
        if hits:
            return st[:max(hits)]
    return st


def exec_depths(asm: str):
    """(function, mnemonic, depth) for every MFMA and vector store: depth is
    the number of exec narrowings that may be in force there, from a
    dataflow over the kernel's control-flow graph (at a join the deeper
    stack is kept, so the answer is conservative)."""
    out = []
    for fn, lines in functions(asm).items():
        bl = basic_blocks(lines)
        state, work = {0: ()}, [0]
        while work:
            i = work.pop()
            st = state[i]
            for l in bl[i]["ins"]:
                st = step(st, l)
            for s in bl[i]["succ"]:
                old = state.get(s)
                if old is None or (depth(st) > depth(old) and depth(st) <= 16):
                    state[s] = st
                    work.append(s)
        for i, b in enumerate(bl):
            st = state.get(i, ())
            for l in b["ins"]:
                st = step(st, l)
                if l.startswith("v_mfma") or re.match(r"(global|buffer)_store", l):
                    out.append((fn, l.split()[0], depth(st)))
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
@pytest.mark.parametrize("src", SRCS, ids=os.path.basename)
def test_mfma_under_full_exec(tmp_path, src):
    rows = exec_depths(device_asm(src, tmp_path))
    mfma = [x for x in rows if x[1].startswith("v_mfma")]
    assert len(mfma) > 0, "no MFMA found in the device code"
    masked = [x for x in mfma if x[2] > 0]
    assert not masked, f"MFMAs under a narrowed exec mask: {masked[:5]}"
    # the same scan sees the lane-conditional stores, so it does see narrowing
    assert any(d > 0 for _, m, d in rows if "store" in m), "the scan found no narrowed region at all"


def _fake_kernel(body: str) -> str:
    return "_Z4fakev:\n" + "\n".join("\t" + l.strip() for l in body.strip().splitlines()) + "\n.Lfunc_end0:\n"


@pytest.mark.parametrize("form", ["saveexec", "written_out"])
def test_scan_sees_both_narrowing_forms(form):
    """The scan on hand-made code: an MFMA inside a lane-dependent loop is
    found narrowed in either form the compiler writes the narrowing, and
    MFMAs before it and after the restore are not."""
    if form == "saveexec":
        enter = "s_and_saveexec_b64 s[4:5], vcc"
    else:
        enter = "s_mov_b64 s[4:5], exec\ns_and_b64 s[6:7], s[4:5], vcc\ns_mov_b64 exec, s[6:7]"
    asm = _fake_kernel(f"""
        v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]
        {enter}
        s_cbranch_execz .LBB0_3
        s_mov_b64 s[8:9], 0
        .LBB0_2:
        v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]
        global_store_dwordx4 v[12:13], v[0:3], off
        s_or_b64 s[8:9], vcc, s[8:9]
        s_andn2_b64 exec, exec, s[8:9]
        s_cbranch_execnz .LBB0_2
        .LBB0_3:
        s_or_b64 exec, exec, s[4:5]
        v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]
        s_endpgm
    """)
    d = [x[2] for x in exec_depths(asm) if x[1].startswith("v_mfma")]
    assert d[0] == 0 and d[1] > 0 and d[2] == 0, d
