"""The library from a C host program on the GPU: tests/c/c_client (built by
__graft_entry__.build() with gcc against include/ and the HIP runtime's C
API, no Python) runs mla_post on a dense split-KV batch read from a file.
Its core must equal the Python binding's bit for bit on the same inputs,
and the small case is checked against the oracle (T4)."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import criteria as C
import oracle.post as O
import synth
from gpu_support import device_inputs, run_debug

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c", "c_client")


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def write_inputs(path, w, codes, scales):
    assert tuple(w.o_strides) == (w.S * 6144, 6144, 512), "the client reads dense partials"
    with open(path, "wb") as f:
        np.array([w.n, w.S], dtype=np.int32).tofile(f)
        np.ascontiguousarray(w.o_buf).view(np.uint16).tofile(f)
        np.ascontiguousarray(w.lse_buf, dtype=np.float32).tofile(f)
        np.ascontiguousarray(codes, dtype=np.uint8).tofile(f)
        np.ascontiguousarray(scales, dtype=np.uint8).tofile(f)
        np.ascontiguousarray(w.gate).view(np.uint16).tofile(f)


@pytest.mark.parametrize(
    "make",
    [lambda: synth.split_merge(), lambda: synth.dense_splits("c_client_persistent", 4, 1040, seed=62, p_neg_inf=0.1)],
    ids=["small", "persistent"],
)
def test_c_client_matches_binding(gpu_lib, tmp_path, make):
    assert os.path.exists(CLIENT), "tests/c/c_client is not built: run __graft_entry__.build()"
    w = make()
    say(f"C client: {w.name} n={w.n} S={w.S}")
    codes, scales = O.quantize_mxfp4(w.wv_bits)
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "core.bin")
    write_inputs(fin, w, codes, scales)
    r = subprocess.run([CLIENT, fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"c_client failed: {r.stdout}{r.stderr}"
    core_c = np.fromfile(fout, dtype=np.uint16).reshape(w.S, 1536)

    d = device_inputs(w, w_codes=codes, w_scales=scales)
    g = run_debug(gpu_lib, d)
    assert np.array_equal(core_c, g["core"]), "C client and Python binding disagree"
    if w.S <= 256:
        ref = O.mla_post(w.o_view(), w.lse_view(), codes, scales, w.gate)
        st = C.check_t4(core_c, ref, g["lat"], g["codes"], g["scales"])
        say(f"C client: {w.name} T4 {st}")
