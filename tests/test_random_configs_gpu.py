"""Seeded random configurations against the oracle, on the GPU.

The explicit cases elsewhere reach every kernel instance one at a time; this
sweep draws shapes, layouts, LSE distributions and masks together, so that
the host's routing boundaries (the one-tile instance with 8- or 16-token
tiles and 8 or 16 rows held per token, the persistent kernel with one or
several tiles per workgroup and 1 to 4 LSE chunks) meet ragged sizes, dead
and poisoned rows, padded and request-major layouts in combinations nobody
wrote by hand. Each case checks T1-T4 on every token; every case is named
(seed, kind, n, S) before it runs.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import criteria as C
import oracle.post as O
import synth
from gpu_support import device_inputs, run_debug

pytestmark = pytest.mark.gpu

CASES = 64
MAX_ROWS = 6500  # n * S cap: each case generates and checks in about a second


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def draw_S(rng) -> int:
    """Token counts on both sides of the routing boundaries at 256 CUs:
    8-token tiles up to 512, 16-token tiles or the persistent kernel up to
    1024, 40 workgroups per head up to 1536, 64 and several tiles each past
    it (and the one-tile instance at any size for one or two partials)."""
    band = rng.choice(5, p=[0.25, 0.25, 0.2, 0.15, 0.15])
    lo, hi = [(1, 64), (65, 512), (513, 1024), (1025, 1536), (1537, 2100)][band]
    return int(rng.integers(lo, hi + 1))


def draw_n(rng) -> int:
    band = rng.choice(5, p=[0.15, 0.35, 0.25, 0.15, 0.10])
    lo, hi = [(1, 1), (2, 8), (9, 16), (17, 64), (65, 200)][band]
    return int(rng.integers(lo, hi + 1))


def make_case(i: int):
    """Case i: a workload and, for request-major layouts, the oracle's
    logical inputs (per-token partials and masked LSEs)."""
    rng = np.random.default_rng(5000 + i)
    kind = str(rng.choice(["dense", "dense", "dense", "dcp", "single", "rm_compact", "rm_page"]))
    seed = 6000 + i
    if kind == "single":
        S = draw_S(rng)
        return synth.single_partial(f"rand{i}_single", S, seed, o_sigma=float(rng.choice([0.5, 1.0, 40.0]))), None
    if kind == "dcp":
        R = int(rng.integers(2, 9))
        S = min(draw_S(rng), MAX_ROWS // R)
        pad = int(rng.integers(0, 9))
        dead_from = int(rng.integers(0, S + 1))
        return synth.dcp_gathered(f"rand{i}_dcp", R, S, seed, head_stride_rows=R * 12 + pad, dead_from=dead_from), None
    if kind.startswith("rm"):
        q = int(rng.choice([1, 2, 4, 8]))
        per = int(rng.integers(1, 17))
        if kind == "rm_page":  # one [per * R, S, 12, 512] tensor: kept small
            per = min(per, 8)
            S = q * int(rng.integers(1, 32 // q + 1))
        else:
            S = q * max(1, min(draw_S(rng), MAX_ROWS // per) // q)
        R = S // q
        batch_rows = int(rng.integers(0, S + 1)) if rng.random() < 0.5 else None
        w = synth.request_major(
            f"rand{i}_{kind}", per=per, q=q, S=S, seed=seed, compact=(kind == "rm_compact"),
            p_neg_inf=float(rng.uniform(0.0, 0.5)), kv_zero=float(rng.choice([0.0, 0.2, 0.6])), batch_rows=batch_rows,
        )
        lse = O.push_mask(w.notes["lse_logical"], w.q, w.kv_lens, w.qsl)
        return w, (w.notes["o_logical"], lse)
    n = draw_n(rng)
    S = min(draw_S(rng), max(1, MAX_ROWS // n))
    p_neg = float(rng.uniform(0.0, 0.6))
    p_nan = float(rng.choice([0.0, 0.05]))
    p_inf = float(rng.choice([0.0, 0.05]))
    if rng.random() < 0.5:
        lse_kw = {"lse_uniform": (-4.0, 16.0)}
    else:
        lse_kw = {"lse_uniform": None, "lse_normal": (float(rng.uniform(-5, 10)), float(rng.choice([1.0, 6.0, 40.0])))}
    return (
        synth.dense_splits(
            f"rand{i}_dense", n, S, seed, o_sigma=float(rng.choice([0.5, 2.0, 30.0])),
            p_neg_inf=p_neg, p_nan=p_nan, p_pos_inf=p_inf, **lse_kw,
        ),
        None,
    )


@pytest.mark.parametrize("i", range(CASES))
def test_random_config(gpu_lib, i):
    w, logical = make_case(i)
    say(f"case {i}: {w.name} n={w.n} S={w.S} q={w.q} masks={w.kv_lens is not None, w.qsl is not None}")
    d = device_inputs(w)
    g = run_debug(gpu_lib, d)
    if logical is None:
        o, lse = w.o_view(), w.lse_view()
    else:
        o, lse = logical
    exact = w.lse_buf is None
    st = C.check_all(o, lse, d["w_codes"], d["w_scales"], w.gate, g, exact_t1=exact, strict_t4=exact)
    assert np.all(np.isfinite(O.bf16_to_f64(g["core"])))
    say(f"case {i}: all {w.S} tokens {st}")
