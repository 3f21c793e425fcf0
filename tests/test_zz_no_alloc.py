"""mla_decode_noalloc (include/mla_decode.h): the fused decode launch with the
library's own scratch array as workspace, for callers that cannot allocate.
Its core equals mla_decode's with a caller workspace, bit for bit, on two
calls in a row, the second smaller than the first (the array keeps the first
call's contents; the counters are cleared by each call), and a call too
large for the array is refused without launching."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.post as O
import synth
from gpu_support import bf16_to_dev, to_bits

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def tensors(d):
    wc, ws = O.quantize_mxfp4(d.wv_bits)
    kv = d.kv if d.kv.shape[0] else np.zeros((1, 576), np.uint16)
    return (bf16_to_dev(d.qry, "cuda"), bf16_to_dev(kv, "cuda"), torch.from_numpy(d.indptr).cuda(), d.q, d.n, d.scale,
            torch.from_numpy(wc).cuda(), torch.from_numpy(ws).cuda(), bf16_to_dev(d.gate, "cuda"))


def test_noalloc_matches_workspace_call(gpu_lib):
    m = gpu_lib
    first = synth.decode_inputs("noalloc_first", [300, 17, 0, 129, 64, 250, 33, 90, 200, 5], 4, 6, seed=80)
    second = synth.decode_inputs("noalloc_second", [40, 77, 3], 2, 3, seed=81)
    for d in (first, second):
        say(f"noalloc: R={d.R} q={d.q} n={d.n}")
        t = tensors(d)
        ws = m.DecodeWorkspace(d.R, d.q, d.n)
        ref = to_bits(m.mla_decode(*t, ws))
        got = to_bits(m.mla_decode_noalloc(*t))
        torch.cuda.synchronize()
        assert np.array_equal(got, ref), f"{d.name}: noalloc core differs from the workspace call"


def test_noalloc_refuses_oversize(gpu_lib):
    m = gpu_lib
    say("noalloc: oversize refused")
    R, q, n = 1024, 4, 16  # 808 MB of partials > 64 MiB
    assert m.decode_workspace_layout(R, q, n)["bytes"] > m.DECODE_SCRATCH_BYTES
    qry = torch.zeros((R * q, 12, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 576), dtype=torch.bfloat16, device="cuda")
    indptr = torch.zeros(R + 1, dtype=torch.int32, device="cuda")
    w_v = torch.zeros((12, 128, 256), dtype=torch.uint8, device="cuda")
    w_s = torch.full((12, 128, 16), 127, dtype=torch.uint8, device="cuda")
    gate = torch.zeros((R * q, 1536), dtype=torch.bfloat16, device="cuda")
    core = torch.full((R * q, 1536), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MlaPostError) as e:
        m.mla_decode_noalloc(qry, kv, indptr, q, n, 0.1, w_v, w_s, gate, core)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((core == 7.0).all()), "a refused call wrote core"
