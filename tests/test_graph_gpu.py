"""mla_post inside a captured HIP graph (GPU): one prepared call is captured
once and replayed several times, with eager work and synchronisations between
the replays; every replay must equal the eager call bit for bit, and a replay
after the inputs changed in place must equal an eager call on the new inputs
(the graph reads the buffers, it holds no copy). Both kernel instances: the
one-tile-per-workgroup instance (small batch) and the persistent one (a
ragged batch of 1100 tokens). The library's launch records no memset."""

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
    "make",
    [
        lambda: synth.dense_splits("graph_small", 8, 128, seed=60),
        lambda: synth.dense_splits("graph_persistent", 16, 1100, seed=61, p_neg_inf=0.05),
    ],
    ids=["small", "persistent"],
)
def test_graph_replays_match_eager(gpu_lib, make):
    m = gpu_lib
    w = make()
    say(f"graph capture: {w.name} n={w.n} S={w.S}")
    d = device_inputs(w)
    core = torch.empty((w.S, 1536), dtype=torch.bfloat16, device="cuda")
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
