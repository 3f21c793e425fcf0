"""The library's launches inside a captured HIP graph (GPU): one prepared call
is captured once and replayed several times, with eager work and
synchronisations between the replays; every replay must equal the eager call
bit for bit, and a replay after the inputs changed in place must equal an
eager call on the new inputs (the graph reads the buffers, it holds no copy).
mla_post's four kernels: the one-tile-per-workgroup kernel (small batch), the
persistent one (a ragged batch of 1100 tokens), the split-rows one (64
splits of 16 tokens) and the streaming one (one partial over 2000 tokens).
The fused decode, with a caller workspace and with the library's own
scratch array (mla_decode_noalloc, whose counter-clearing fill kernel is
captured with it): its counters must be back at zero after every replay.
o_proj (1000 tokens, D = 7168). No launch records a memset."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_support import device_inputs, to_bits

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize(
    "make,kernel",
    [
        (lambda: synth.dense_splits("graph_small", 8, 128, seed=60), "one_tile"),
        (lambda: synth.dense_splits("graph_persistent", 16, 1100, seed=61, p_neg_inf=0.05), "persistent"),
        (lambda: synth.dense_splits("graph_split_rows", 64, 16, seed=62, p_neg_inf=0.05), "split_rows"),
        (lambda: synth.dense_splits("graph_stream", 1, 2000, seed=63, p_neg_inf=0.05), "stream"),
    ],
    ids=["small", "persistent", "split_rows", "stream"],
)
def test_graph_replays_match_eager(gpu_lib, make, kernel):
    m = gpu_lib
    w = make()
    say(f"graph capture: {w.name} n={w.n} S={w.S}")
    d = device_inputs(w)
    core = torch.empty((w.S, 1536), dtype=torch.bfloat16, device="cuda")
    assert m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core)["kernel"] == kernel
    call = m.prepare(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core)
    call()
    torch.cuda.synchronize()
    eager = to_bits(core)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture's stream kind, outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        core.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(core), eager), f"replay {rep} differs from the eager call"

    # new inputs in place: gate x 2 (power of two, so core doubles exactly)
    d["gate"].mul_(2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = to_bits(core)
    call()
    torch.cuda.synchronize()
    assert np.array_equal(replayed, to_bits(core)), "replay on changed inputs differs from the eager call"
    doubled = (torch.from_numpy(eager.view(np.int16)).view(torch.bfloat16).float() * 2).to(torch.bfloat16)
    assert np.array_equal(replayed, doubled.view(torch.int16).numpy().view(np.uint16))
    say(f"graph capture: {w.name} ok")


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture's stream kind, outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_decode_graph_replays_match_eager(gpu_lib, noalloc):
    import oracle.post as O
    from gpu_support import bf16_to_dev

    m = gpu_lib
    d = synth.decode_inputs("graph_decode", [300, 17, 0, 129, 64, 250, 33, 90, 200, 5, 400, 77], 4, 5, seed=64)
    say(f"graph capture: decode R={d.R} q={d.q} n={d.n} noalloc={noalloc}")
    wc, wsc = O.quantize_mxfp4(d.wv_bits)
    qry, kv = bf16_to_dev(d.qry, "cuda"), bf16_to_dev(d.kv, "cuda")
    indptr = torch.from_numpy(d.indptr).cuda()
    w_v, w_s = torch.from_numpy(wc).cuda(), torch.from_numpy(wsc).cuda()
    gate = bf16_to_dev(d.gate, "cuda")
    core = torch.empty((d.R * d.q, 1536), dtype=torch.bfloat16, device="cuda")
    ws = m.DecodeWorkspace(d.R, d.q, d.n)
    args = (qry, kv, indptr, d.q, d.n, d.scale, w_v, w_s, gate)
    if noalloc:
        def call():
            m.mla_decode_noalloc(*args, core)
    else:
        fused = m.PreparedDecode(qry, kv, indptr, d.q, d.n, d.scale, w_v, w_s, gate, ws, core, fused=True)

        def call():
            fused()
    call()
    torch.cuda.synchronize()
    eager = to_bits(core)
    g = _capture(call)
    for rep in range(3):
        core.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(core), eager), f"replay {rep} differs from the eager call"
        if not noalloc:
            cnt = ws.counters().cpu().numpy()
            assert np.all(cnt == 0), f"replay {rep} left counters at {cnt[cnt != 0][:8]}"
    gate.mul_(2)  # power of two: core doubles exactly
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = to_bits(core)
    call()
    torch.cuda.synchronize()
    assert np.array_equal(replayed, to_bits(core)), "replay on changed inputs differs from the eager call"
    say(f"graph capture: decode noalloc={noalloc} ok")


def test_oproj_graph_replays_match_eager(gpu_lib):
    m = gpu_lib
    rng = np.random.default_rng(65)
    S, D, K = 1000, 7168, 1536
    say(f"graph capture: oproj S={S} D={D} K={K} plan={m.oproj_plan(S, D)}")
    core = torch.from_numpy(synth.f32_to_bf16_bits(rng.standard_normal((S, K), dtype=np.float32)).view(np.int16))
    core = core.view(torch.bfloat16).cuda()
    w = synth.f32_to_bf16_bits(rng.standard_normal((D, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    w = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((S, D), dtype=torch.bfloat16, device="cuda")
    call = m.PreparedOproj(core, w, out)
    call()
    torch.cuda.synchronize()
    eager = to_bits(out)
    g = _capture(call)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), eager), f"replay {rep} differs from the eager call"
    say("graph capture: oproj ok")
