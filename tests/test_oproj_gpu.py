"""o_proj (include/mla_oproj.h) on the GPU against the float64 oracle
(oracle/oproj.py), through the C ABI: criterion T5 on every output.

Inputs are seeded and synthetic: core ~ N(0, 1) bf16 (or the core that
mla_post produced for a standard workload), W_O ~ N(0, 1/sqrt(K)) bf16.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import criteria as C
import oracle.post as O
import synth
from gpu_support import bf16_to_dev, device_inputs, to_bits
from oracle.oproj import oproj as oracle_oproj

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def check(m, core_bits, w_bits, rows_per_chunk=1024):
    S, K = core_bits.shape
    D = w_bits.shape[0]
    core = bf16_to_dev(core_bits, "cuda")
    w = bf16_to_dev(w_bits, "cuda")
    out = m.oproj(core, w)
    torch.cuda.synchronize()
    g = to_bits(out)
    st = {}
    for r0 in range(0, S, rows_per_chunk):
        rows = np.arange(r0, min(S, r0 + rows_per_chunk))
        ref = oracle_oproj(core_bits, w_bits, rows=rows)
        s = C.check_t5(g[rows], ref, K)
        st["t5_exact_frac"] = min(st.get("t5_exact_frac", 1.0), s["t5_exact_frac"])
        st["t5_max_err_over_bound"] = max(st.get("t5_max_err_over_bound", 0.0), s["t5_max_err_over_bound"])
    return g, st


@pytest.mark.parametrize(
    "S,D,K",
    [
        (4096, 7168, 1536),  # the large decode batch's core into a 7168-wide o_proj
        (4000, 7000, 1536),  # 256 x 256 tiles, ragged in both dimensions
        (2600, 6664, 960),  # 256 x 256 tiles, an odd number of K steps of 64
        (4096, 4096, 1536),  # 256 x 256 tiles, one round on 256 CUs
        (3900, 4000, 704),  # 256 x 256 tiles, ragged in both dimensions, 11 K steps of 64
        (1, 7168, 1536),
        (37, 7168, 1536),  # ragged token tile, small-batch tiling
        (300, 1024, 1536),  # between tilings
        (129, 136, 1536),  # ragged output tile (D not a multiple of 64)
        (5, 8, 64),  # the smallest D and K
        (700, 264, 640),
    ],
    ids=lambda v: str(v),
)
def test_oproj_parity(gpu_lib, S, D, K):
    rng = np.random.default_rng(S * 7 + D + K)
    core = synth.f32_to_bf16_bits(rng.standard_normal((S, K), dtype=np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((D, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    say(f"oproj S={S} D={D} K={K} plan={gpu_lib.oproj_plan(S, D)}")
    _, st = check(gpu_lib, core, w)
    say(f"oproj S={S} D={D} K={K}: {st}")


def test_oproj_strided_and_canary(gpu_lib):
    """core as a column slice of a wider buffer and out as a slice of a
    wider, canary-filled buffer: only out[:S, :D] is written, equal to the
    dense call's result."""
    m = gpu_lib
    rng = np.random.default_rng(3)
    S, D, K = 77, 200, 1536
    core = synth.f32_to_bf16_bits(rng.standard_normal((S, K), dtype=np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((D, K), dtype=np.float32) / np.float32(40.0))
    say("oproj strided + canary")
    dense = to_bits(m.oproj(bf16_to_dev(core, "cuda"), bf16_to_dev(w, "cuda")))
    wide = torch.zeros((S, K + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, 32 : 32 + K] = bf16_to_dev(core, "cuda")
    buf = torch.full((S + 2, D + 16), 0, dtype=torch.int16, device="cuda")
    buf.fill_(0x7E57)
    out = buf[1 : S + 1, 8 : 8 + D].view(torch.bfloat16)
    m.oproj(wide[:, 32 : 32 + K], bf16_to_dev(w, "cuda"), out)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert np.array_equal(h[1 : S + 1, 8 : 8 + D], dense)
    assert np.all(h[0] == 0x7E57) and np.all(h[-1] == 0x7E57)
    assert np.all(h[:, :8] == 0x7E57) and np.all(h[:, 8 + D :] == 0x7E57)


def test_oproj_after_mla_post(gpu_lib):
    """The path and its consumer on one stream: mla_post's core of the
    decode-context-parallel workload feeds o_proj (D = 7168); the result
    meets T5 against the oracle run on that core, and tokens whose partials
    are all empty (rows 240 on) give exact zeros."""
    m = gpu_lib
    w = synth.dcp8()
    d = device_inputs(w)
    rng = np.random.default_rng(11)
    D = 7168
    wo = synth.f32_to_bf16_bits(rng.standard_normal((D, 1536), dtype=np.float32) / np.float32(np.sqrt(1536)))
    say("mla_post -> oproj, dcp8")
    core = m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"])
    out = m.oproj(core, bf16_to_dev(wo, "cuda"))
    torch.cuda.synchronize()
    cb = to_bits(core)
    ref = oracle_oproj(cb, wo)
    C.check_t5(to_bits(out), ref, 1536)
    assert np.all(to_bits(out)[240:] == 0)


def test_oproj_empty_and_errors(gpu_lib):
    m = gpu_lib
    say("oproj S=0 and argument errors")
    core = torch.zeros((0, 1536), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 1536), dtype=torch.bfloat16, device="cuda")
    out = m.oproj(core, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
    with pytest.raises(m.MlaPostError):
        m.oproj(torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda"), torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda"))
