"""The streaming kernel (one or two partials per (token, head) over many
tokens; MLA_POST_KERNEL_STREAM in mla_post.h) on the GPU, through the C ABI,
against the oracle: T1-T4 on every token of every case, plus the checks that
every core row is written (a NaN-filled core comes back finite and equal to
the first call's) and that the plan routes each case to this kernel.

Cases: dense partials with -inf / NaN / +inf LSEs at ragged sizes, one
partial without LSEs, strided (gathered, padded) head layouts, the
request-major layout with tokens past the batch, and a long case where each
workgroup walks about 30 tiles (so the loop over three LDS buffers wraps
many times and ends at every phase across the workgroups).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import criteria as C
import oracle.post as O
import synth
from gpu_support import device_inputs, run_debug, to_bits

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def run_case(m, w, reference=None):
    say(f"{w.name}: n={w.n} S={w.S} q={w.q} strides={w.o_strides} o_sr={w.o_sr}")
    d = device_inputs(w)
    p = m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], **d["layout"])
    assert p["kernel"] == "stream" and p["tile_tokens"] == 16 // w.n and p["rows_held"] == w.n, p
    g = run_debug(m, d)
    core = torch.full((w.S, 1536), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core, **d["layout"])
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core), g["core"]), "a second call (no stage outputs) differs"
    assert bool(torch.isfinite(core.float()).all()), "a core row was not written"
    if reference is None:
        st = C.check_all(w.o_view(), w.lse_view(), d["w_codes"], d["w_scales"], w.gate, g,
                         exact_t1=w.lse_buf is None)
    else:
        ref = reference(w, d)
        st = {}
        st.update(C.check_t1(g["lat"], ref))
        st.update(C.check_t2(g["lat"], g["codes"], g["scales"]))
        st.update(C.check_t3(g["core"], g["codes"], g["scales"], d["w_codes"], d["w_scales"], w.gate))
        st.update(C.check_t4(g["core"], ref, g["lat"], g["codes"], g["scales"]))
    say(f"{w.name}: plan {p}; {st}")
    return g, p


DENSE = [
    # one partial with LSEs: dead (-inf), NaN and +inf LSEs give +0 latents
    ("n1_S4099", 1, 4099, 70, dict(p_neg_inf=0.1, p_nan=0.01, p_pos_inf=0.01)),
    # the smallest batch the plan streams, at 256 CUs (6 tokens per CU)
    ("n1_S1536", 1, 1536, 71, dict(p_neg_inf=0.05)),
    ("n2_S3001", 2, 3001, 72, dict(p_neg_inf=0.2, p_nan=0.01, p_pos_inf=0.01)),
    ("n2_S1541", 2, 1541, 73, dict(p_neg_inf=0.05)),
    # about 30 tiles per workgroup
    ("n1_S20000", 1, 20000, 74, dict(p_neg_inf=0.05)),
    ("n2_S10007", 2, 10007, 75, dict(p_neg_inf=0.05, lse_normal=(8.0, 6.0))),
]


@pytest.mark.parametrize("name,n,S,seed,opts", DENSE, ids=[c[0] for c in DENSE])
def test_stream_dense(gpu_lib, name, n, S, seed, opts):
    w = synth.dense_splits(name, n, S, seed=seed, **opts)
    g, _ = run_case(gpu_lib, w)
    # (token, head) pairs all of whose partials are dead: exact +0 latents
    lse = w.lse_view()
    dead = ~np.any(np.isfinite(lse) & (lse != np.inf), axis=0)  # [S, 12]
    assert np.all(g["lat"][dead] == 0)


def test_stream_one_partial_no_lse(gpu_lib):
    w = synth.single_partial("stream_nolse_S5003", 5003, seed=76)
    run_case(gpu_lib, w)


@pytest.mark.parametrize("R", [1, 2], ids=["one_rank", "two_ranks"])
def test_stream_gathered_heads(gpu_lib, R):
    """Decode-context-parallel partials gathered with a padded head stride
    (NaN in the padding, never read), one or two ranks."""
    w = synth.dcp_gathered(f"stream_dcp{R}", R, 3100, seed=77 + R, head_stride_rows=R * 12 + 5, dead_from=3050)
    g, _ = run_case(gpu_lib, w)
    assert np.all(g["core"][3050:] == 0) and np.all(g["lat"][3050:] == 0)


def _request_major_reference(w, d):
    lse = O.push_mask(w.notes["lse_logical"], w.q, w.kv_lens, w.qsl)
    return O.mla_post(w.notes["o_logical"], lse, d["w_codes"], d["w_scales"], w.gate)


def test_stream_request_major_past_batch(gpu_lib):
    """Request-major slices of one split ([R, 1, q, 12, 512], q = 4: rows
    move by a fixed stride per token) with the batch ending 13 tokens before
    S: those tokens' core rows are exactly +0."""
    S = 3200
    w = synth.request_major("stream_rm1", per=1, q=4, S=S, seed=81, compact=True, batch_rows=S - 13)
    g, _ = run_case(gpu_lib, w, reference=_request_major_reference)
    assert np.all(g["core"][S - 13:] == 0) and np.all(g["lat"][S - 13:] == 0)


def test_request_major_two_splits_not_streamed(gpu_lib):
    """Two splits request-major ([R, 2, q, 12, 512]) have a request offset
    per token: the plan leaves them to the one-tile kernel; T1-T4 hold."""
    m = gpu_lib
    S = 3200
    w = synth.request_major("rm2_not_streamed", per=2, q=4, S=S, seed=82, compact=True, batch_rows=S - 13)
    d = device_inputs(w)
    p = m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], **d["layout"])
    assert p["kernel"] == "one_tile", p
    g = run_debug(m, d)
    ref = _request_major_reference(w, d)
    st = {}
    st.update(C.check_t1(g["lat"], ref))
    st.update(C.check_t2(g["lat"], g["codes"], g["scales"]))
    st.update(C.check_t3(g["core"], g["codes"], g["scales"], d["w_codes"], d["w_scales"], w.gate))
    st.update(C.check_t4(g["core"], ref, g["lat"], g["codes"], g["scales"]))
    say(f"{w.name}: plan {p}; {st}")
    assert np.all(g["core"][S - 13:] == 0)
