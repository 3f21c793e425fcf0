"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Every input is seeded and synthetic (synth.workloads); W_V is put into MXFP4
by the oracle's quantiser. Stage outputs (latents, codes, scales) come from
the same kernel launch as core. Criteria T1-T4 are defined in criteria.py.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import criteria as C
import oracle.post as O
import synth
from gpu_support import bf16_to_dev, device_inputs, run_debug, to_bits

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def full_parity(m, w, strict_t4=False):
    """Run w on the GPU with stage outputs and check T1-T4 on every token;
    returns the statistics."""
    say(f"{w.name}: n={w.n} S={w.S} strides={w.o_strides}")
    d = device_inputs(w)
    g = run_debug(m, d)
    stats = C.check_all(w.o_view(), w.lse_view(), d["w_codes"], d["w_scales"], w.gate, g,
                        exact_t1=w.lse_buf is None, strict_t4=strict_t4)
    say(f"{w.name}: {stats}")
    return stats, g, d


# ---------------------------------------------------------------- the five standard workloads


def test_tiny(gpu_lib):
    full_parity(gpu_lib, synth.tiny(), strict_t4=True)


def test_no_merge(gpu_lib):
    full_parity(gpu_lib, synth.no_merge(), strict_t4=True)


def test_split_merge(gpu_lib):
    full_parity(gpu_lib, synth.split_merge())


def test_dcp8(gpu_lib):
    stats, g, _ = full_parity(gpu_lib, synth.dcp8())
    # tokens >= 240 have every LSE -inf: exact zeros
    assert np.all(g["core"][240:] == 0) and np.all(g["lat"][240:] == 0)


def test_large_decode_full(gpu_lib):
    """Full-size large decode batch (805 MB of partials), launched as the
    benchmark launches it (no stage outputs) and with stage outputs: core is
    bit-identical between the two, and T1-T4 hold on every one of the 4096
    tokens (all 786k blocks for T2)."""
    m = gpu_lib
    w = synth.large_decode()
    say(f"{w.name}: n={w.n} S={w.S}")
    d = device_inputs(w)
    core_plain = m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"])
    torch.cuda.synchronize()
    g = run_debug(m, d)
    assert np.array_equal(to_bits(core_plain), g["core"]), "stage outputs changed core"
    st = C.check_all(w.o_view(), w.lse_view(), d["w_codes"], d["w_scales"], w.gate, g)
    say(f"{w.name}: all tokens {st}")


@pytest.mark.parametrize(
    "make",
    [
        # a second 64-lane LSE chunk holding 2 splits
        pytest.param(lambda: synth.dense_splits("persistent_n66", 66, 1040, seed=25, p_neg_inf=0.2), id="n66_S1040"),
        # decode-context-parallel gathered partials, 8 ranks, padded head stride
        pytest.param(lambda: synth.dcp_gathered("persistent_dcp8", 8, 1100, seed=26, head_stride_rows=104, dead_from=1090),
                     id="dcp8_S1100"),
        # more than 8 tiles per workgroup (S > 8 x 64 x 16): the staged output
        # is written after 8 tiles and its buffers reused for the rest
        pytest.param(lambda: synth.dense_splits("persistent_long", 2, 9000, seed=27, p_neg_inf=0.1), id="n2_S9000"),
        # 4 and 8 LSE chunks in the persistent kernel (with fewer tokens these
        # many splits take the split-rows kernel)
        pytest.param(lambda: synth.dense_splits("persistent_n129", 129, 340, seed=44, p_neg_inf=0.2), id="n129_S340"),
        pytest.param(lambda: synth.dense_splits("persistent_n257", 257, 340, seed=45, p_neg_inf=0.3), id="n257_S340"),
    ],
)
def test_persistent_multi_tile(gpu_lib, make):
    """The persistent kernel with several token tiles per workgroup (S past
    1024, so tiles i and i + 64 share a workgroup and the software pipeline
    runs across them), a ragged last tile and the short tiles the leftover
    tokens are dealt out as: T1-T4 on every token."""
    m = gpu_lib
    w = make()
    say(f"{w.name}: n={w.n} S={w.S}")
    d = device_inputs(w)
    g = run_debug(m, d)
    # every row is written: a NaN-filled core comes back finite and equal to
    # the first call's, bit for bit
    core = torch.full((w.S, 1536), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core, **d["layout"])
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core), g["core"])
    assert bool(torch.isfinite(core.float()).all())
    st = C.check_all(w.o_view(), w.lse_view(), d["w_codes"], d["w_scales"], w.gate, g)
    say(f"{w.name}: all tokens {st}")


# ---------------------------------------------------------------- edge cases


@pytest.mark.parametrize(
    "w",
    [
        pytest.param(lambda: synth.dense_splits("ragged_S37", 3, 37, seed=10, p_neg_inf=0.2), id="ragged_S37"),
        pytest.param(lambda: synth.dense_splits("S1", 5, 1, seed=15), id="S1"),
        pytest.param(lambda: synth.dense_splits("n1_with_lse", 1, 19, seed=13, p_neg_inf=0.3, p_nan=0.1, p_pos_inf=0.1), id="n1_lse"),
        # 16 splits on 8-token tiles: the one-tile instance holding 16 rows per token
        pytest.param(lambda: synth.dense_splits("n16_small", 16, 50, seed=31, p_neg_inf=0.2), id="n16_one_tile"),
        # more than 64 splits and few tokens: the split-rows kernel, one token
        # per workgroup, 2, 4 and 8 LSE chunks
        pytest.param(lambda: synth.dense_splits("n65", 65, 9, seed=11, p_neg_inf=0.1), id="n65_two_chunks"),
        pytest.param(lambda: synth.dense_splits("n200", 200, 5, seed=30, p_neg_inf=0.3), id="n200_four_chunks"),
        pytest.param(lambda: synth.dense_splits("n300", 300, 3, seed=12, p_neg_inf=0.5), id="n300_eight_chunks"),
        pytest.param(lambda: synth.dense_splits("nmax", 512, 2, seed=16, p_neg_inf=0.05), id="n_max_512"),
        pytest.param(lambda: synth.dense_splits("all_dead", 4, 20, seed=14, p_neg_inf=1.0), id="all_dead"),
        pytest.param(lambda: synth.dense_splits("wide_lse", 12, 24, seed=17, lse_normal=(0.0, 80.0)), id="wide_lse_spread"),
        pytest.param(lambda: synth.dcp_gathered("dcp3_pad", 3, 29, seed=18, head_stride_rows=40, dead_from=20), id="dcp3_padded"),
        pytest.param(lambda: synth.single_partial("no_merge_S5", 5, seed=19, o_sigma=300.0), id="no_merge_ragged"),
        # the one-tile instance at 256 CUs: 8-token tiles up to S = 512 (with
        # 9-16 splits in the 16-row form), 16-token tiles beyond (n <= 8; with
        # more splits that range takes the persistent kernel)
        pytest.param(lambda: synth.dense_splits("latency8_n8", 8, 500, seed=32, p_neg_inf=0.1), id="latency8_n8_S500"),
        pytest.param(lambda: synth.dense_splits("latency8_n16", 16, 510, seed=33, p_neg_inf=0.2), id="latency8_n16_S510"),
        pytest.param(lambda: synth.dense_splits("latency16", 4, 900, seed=28, p_neg_inf=0.1), id="latency16_S900"),
        pytest.param(lambda: synth.single_partial("latency16_no_lse", 700, seed=29), id="latency16_no_lse"),
        # the instances holding 2 and 4 rows per token (n <= 2, n <= 4)
        pytest.param(lambda: synth.dense_splits("latency16_n2", 2, 777, seed=37, p_neg_inf=0.3), id="latency16_n2"),
        pytest.param(lambda: synth.dense_splits("latency8_n4", 4, 300, seed=38, p_neg_inf=0.3, p_nan=0.05),
                     id="latency8_n4"),
        # between one workgroup per CU and 64 tiles per head: every workgroup
        # one short tile (64 per head, two of them with none at S = 800; 40
        # per head, one with none, at S = 345), one full tile each (42 tiles),
        # and one per tile with only the 1-token last tile past the first round
        pytest.param(lambda: synth.dense_splits("n16_S800", 16, 800, seed=34, p_neg_inf=0.2), id="n16_persistent_short_tiles"),
        pytest.param(lambda: synth.dense_splits("n20_S345", 20, 345, seed=40, p_neg_inf=0.2), id="n20_persistent_40_short"),
        pytest.param(lambda: synth.dense_splits("n24_S672", 24, 672, seed=41, p_neg_inf=0.2), id="n24_persistent_42_full"),
        pytest.param(lambda: synth.dense_splits("n40_S337", 40, 337, seed=42, p_neg_inf=0.2), id="n40_persistent_22_tiles"),
        # S past one device-filling wave of workgroups (more than 64 tiles per
        # head at 256 CUs): the persistent kernel, with a ragged last tile
        pytest.param(lambda: synth.dense_splits("persistent_ragged", 3, 1030, seed=23, p_neg_inf=0.2), id="persistent_ragged"),
        pytest.param(lambda: synth.single_partial("persistent_no_lse", 1100, seed=24), id="persistent_no_lse"),
        # one or two partials past S = 1024: the one-tile instance, many rounds
        pytest.param(lambda: synth.dense_splits("big_n1", 1, 2100, seed=35, p_neg_inf=0.2), id="one_tile_large_n1"),
        pytest.param(lambda: synth.dense_splits("big_n2", 2, 1500, seed=36, p_neg_inf=0.3), id="one_tile_large_n2"),
        # 3 or 4 partials past S = 1024: the persistent kernel with both tokens'
        # rows issued a tile ahead
        pytest.param(lambda: synth.dense_splits("pair_n3", 3, 2100, seed=39, p_neg_inf=0.2), id="persistent_pair_n3"),
    ],
)
def test_edge(gpu_lib, w):
    w = w()
    stats, g, _ = full_parity(gpu_lib, w, strict_t4=(w.n <= 1 and w.lse_buf is None))
    if w.name == "all_dead":
        assert np.all(g["core"] == 0) and np.all(g["lat"] == 0) and np.all(g["scales"] == 1)
        assert np.all(g["codes"] == 0)


@pytest.mark.parametrize(
    "n,S",
    [(6, 40), (16, 1100), (20, 400), (66, 340), (3, 1100), (4, 2100), (24, 150), (33, 64), (20, 40), (66, 20)],
    ids=["one_tile_instance", "persistent_n16", "persistent_n20", "persistent_two_chunks", "persistent_pair_n3",
         "persistent_pair_n4", "split_rows_tile8", "split_rows_tile4", "split_rows_tile2", "split_rows_two_chunks"],
)
def test_dead_rows_nan_inf_unused(gpu_lib, n, S):
    """Rows of weight 0 hold NaN and inf: the result equals the oracle's, which
    never touches them, and is finite. Both kernels load some such rows before
    their weights are known (the one-tile instance all of its rows, the
    persistent kernel the first 8 rows of each workgroup's first tile) and
    must leave them out of the sum (the split-rows kernel too: it loads every
    row of its tokens up front)."""
    w = synth.dense_splits(f"poisoned_dead_n{n}", n, S, seed=20, p_neg_inf=0.2, p_nan=0.1, p_pos_inf=0.1)
    lse = w.lse_view()
    dead = ~np.isfinite(lse)
    ob = w.o_buf.copy()
    ob[dead] = np.where(np.arange(512) % 2 == 0, 0x7FC0, 0x7F80).astype(np.uint16)
    w.o_buf = ob
    stats, g, _ = full_parity(gpu_lib, w)
    assert np.all(np.isfinite(O.bf16_to_f64(g["core"])))


# (n, S, tokens per workgroup the plan gives at 256 CUs, workload options):
# every instance (waves per token G = 8 / tile, LSE chunks), ragged last tiles
SPLIT_ROWS = [
    # one wave per token (8-token tiles): a wave streams all of a token's rows,
    # up to 4 batches of 16 (one LSE chunk) or 8 (two)
    (20, 157, 8, dict(p_neg_inf=0.2)),
    (100, 130, 8, dict(p_neg_inf=0.1)),
    # 2 waves per token (4-token tiles): rows j = g, g + 2, ..; 1, 2, 4 chunks
    (33, 64, 4, dict(p_neg_inf=0.1)),
    (64, 43, 4, dict(p_neg_inf=0.05, p_pos_inf=0.05)),
    (100, 61, 4, dict(p_neg_inf=0.2)),
    (200, 50, 4, dict(p_neg_inf=0.3, p_nan=0.05)),
    # 4 waves per token (2-token tiles): n not a multiple of 4; 1, 2, 4, 8 chunks
    (40, 33, 2, dict(p_neg_inf=0.1)),
    (128, 41, 2, dict(p_neg_inf=0.1)),
    (250, 35, 2, dict(p_neg_inf=0.2)),
    (300, 41, 2, dict(p_neg_inf=0.4)),
    # 8 waves per token, one token per workgroup: 1, 2, 4 and 8 chunks
    (50, 10, 1, dict(p_neg_inf=0.2)),
    (100, 7, 1, dict(p_neg_inf=0.1)),
    (129, 3, 1, dict(p_neg_inf=0.1)),
    (300, 2, 1, dict(p_neg_inf=0.4, p_nan=0.05)),
    (512, 1, 1, dict(p_neg_inf=0.02)),
    # tokens all of whose partials are dead: exact zeros
    (24, 150, 8, dict(p_neg_inf=0.9)),
    # past S = 160 with 64 splits or more (up to S = 192)
    (64, 190, 4, dict(p_neg_inf=0.1)),
]


@pytest.mark.parametrize("n,S,tt,opts", SPLIT_ROWS, ids=[f"n{n}_S{S}_tile{tt}" for n, S, tt, _ in SPLIT_ROWS])
def test_split_rows(gpu_lib, n, S, tt, opts):
    """The split-rows kernel (several waves per token, each summing every
    G-th partial, the sums added in LDS): the plan takes it with the expected
    tile, and every token meets T1-T4 against the oracle."""
    m = gpu_lib
    w = synth.dense_splits(f"split_rows_n{n}_S{S}", n, S, seed=100 + n, **opts)
    d = device_inputs(w)
    p = m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"])
    assert p["kernel"] == "split_rows" and p["tile_tokens"] == tt, p
    stats, g, _ = full_parity(m, w)
    # (token, head) pairs all of whose partials are dead: exact +0 latents,
    # zero codes, scale code 1 and +0 core (the gate is non-negative)
    dead = ~np.isfinite(w.lse_view()).any(axis=0)  # [S, 12]
    if dead.any():
        assert np.all(g["lat"][dead] == 0) and np.all(g["codes"][dead] == 0) and np.all(g["scales"][dead] == 1)
        core = g["core"].reshape(w.S, 12, 128)
        assert np.all(core[dead] == 0)
    if opts.get("p_neg_inf", 0) >= 0.9:
        assert dead.sum() > 0, "the all-dead case must hold dead (token, head) pairs"


@pytest.mark.parametrize("S", [300, 1100], ids=["one_tile", "persistent"])
def test_one_partial_with_lse_is_copied(gpu_lib, S):
    """One partial with an LSE is copied, not merged: its weight is 1 or 0.
    A token whose LSE sanitises to -inf (-inf, NaN, +inf) gives exact zeros
    although its row holds NaN and inf; every other token's latents are its
    row bit for bit, except that -0 becomes +0 (as in the merge, whose sum
    starts at +0); T1-T4 hold against the oracle."""
    m = gpu_lib
    w = synth.dense_splits(f"copy_lse_S{S}", 1, S, seed=50, p_neg_inf=0.2, p_nan=0.05, p_pos_inf=0.05)
    dead = ~np.isfinite(w.lse_view()[0])  # [S, 12]
    ob = w.o_buf.copy()
    ob[0][dead] = np.where(np.arange(512) % 2 == 0, 0x7FC0, 0x7F80).astype(np.uint16)
    ob[0][~dead, ::7] = 0x8000  # -0 in live rows
    w.o_buf = ob
    stats, g, _ = full_parity(m, w)
    expect = np.where(dead[..., None], 0, ob[0])
    expect = np.where((expect & 0x7FFF) == 0, 0, expect).astype(np.uint16)
    assert np.array_equal(g["lat"], expect)
    assert np.all(np.isfinite(O.bf16_to_f64(g["core"])))


@pytest.mark.parametrize("n,S", [(4, 33), (20, 33), (20, 400)], ids=["one_tile_instance", "split_rows", "persistent"])
def test_strided_weights_and_lse(gpu_lib, n, S):
    """W_V codes as a column slice of a wider buffer, scales stored with the
    block axis outermost, lse as a non-dense view: same result as the dense
    layout, and equal to the oracle (4 splits: the one-tile instance; 20
    splits: the split-rows kernel at S = 33, the persistent one at 400)."""
    m = gpu_lib
    w = synth.dense_splits("strided", n, S, seed=21, p_neg_inf=0.1)
    d = device_inputs(w)
    base = run_debug(m, d)
    wide = torch.zeros((12, 128, 512), dtype=torch.uint8, device="cuda")
    wide[:, :, 128:384] = d["w_v"]
    w_v = wide[:, :, 128:384]
    sc_t = d["w_v_scale"].permute(2, 0, 1).contiguous()  # [16, 12, 128]
    w_s = sc_t.permute(1, 2, 0)  # logical [12, 128, 16], strides (128, 1, 1536)
    lse_wide = torch.full((n, S, 12, 3), float("nan"), device="cuda")
    lse_wide[..., 1] = d["lse"]
    lse_v = lse_wide[..., 1]
    say("strided: w_v slice, scales block-major, lse stride 3")
    core, lat, codes, scales = m.mla_post(d["o"], lse_v, w_v, w_s, d["gate"], debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core), base["core"])
    assert np.array_equal(to_bits(lat), base["lat"])
    full_parity(m, w)


def test_canary_and_coverage(gpu_lib):
    """core is written for every token < S and nowhere else: rows around it
    keep their canary, and no poisoned element survives inside."""
    m = gpu_lib
    w = synth.dense_splits("canary", 3, 21, seed=22, p_neg_inf=0.1)
    d = device_inputs(w)
    buf = torch.full((w.S + 2, 1536), 0, dtype=torch.int16, device="cuda")
    buf[0] = 0x7E57
    buf[-1] = 0x7E57
    buf[1:-1] = -1  # 0xFFFF, a NaN pattern the kernel never writes
    core = buf[1:-1].view(torch.bfloat16)
    say("canary")
    m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core=core)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert np.all(h[0] == 0x7E57) and np.all(h[-1] == 0x7E57)
    assert not np.any(h[1:-1] == 0xFFFF)


def test_empty_batch_is_noop(gpu_lib):
    m = gpu_lib
    say("S=0")
    o = torch.zeros((2, 0, 12, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 0, 12), dtype=torch.float32, device="cuda")
    w_v = torch.zeros((12, 128, 256), dtype=torch.uint8, device="cuda")
    w_s = torch.full((12, 128, 16), 127, dtype=torch.uint8, device="cuda")
    gate = torch.zeros((0, 1536), dtype=torch.bfloat16, device="cuda")
    core = m.mla_post(o, lse, w_v, w_s, gate)
    torch.cuda.synchronize()
    assert core.shape == (0, 1536)


def test_deterministic(gpu_lib):
    """Two launches give bit-identical core."""
    m = gpu_lib
    w = synth.split_merge()
    d = device_inputs(w)
    say("determinism")
    a = to_bits(m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"]))
    b = to_bits(m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"]))
    assert np.array_equal(a, b)


def test_concurrent_streams(gpu_lib):
    """Calls running at the same time on two streams (default priority) do not
    interfere: the library keeps no device state between or across calls. A
    persistent-kernel call and a one-tile call, and two calls of the same
    workload into different outputs, each equal their serial result."""
    m = gpu_lib
    wa = synth.dense_splits("conc_persistent", 16, 1100, seed=70, p_neg_inf=0.05)
    wb = synth.dense_splits("conc_small", 8, 128, seed=71, p_neg_inf=0.1)
    da, db = device_inputs(wa), device_inputs(wb)
    say("concurrent streams")
    ref_a = to_bits(m.mla_post(da["o"], da["lse"], da["w_v"], da["w_v_scale"], da["gate"]))
    ref_b = to_bits(m.mla_post(db["o"], db["lse"], db["w_v"], db["w_v_scale"], db["gate"]))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.full((wa.S, 1536), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    outs_b = [torch.full((wb.S, 1536), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    outs_a2 = [torch.full((wa.S, 1536), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(4):
        with torch.cuda.stream(s1):
            m.mla_post(da["o"], da["lse"], da["w_v"], da["w_v_scale"], da["gate"], outs_a[i])
        with torch.cuda.stream(s2):
            m.mla_post(db["o"], db["lse"], db["w_v"], db["w_v_scale"], db["gate"], outs_b[i])
            m.mla_post(da["o"], da["lse"], da["w_v"], da["w_v_scale"], da["gate"], outs_a2[i])
    torch.cuda.synchronize()
    for i in range(4):
        assert np.array_equal(to_bits(outs_a[i]), ref_a)
        assert np.array_equal(to_bits(outs_a2[i]), ref_a)
        assert np.array_equal(to_bits(outs_b[i]), ref_b)


def test_ranks_helper_matches_view(gpu_lib):
    """mla_post_ranks on the gathered [S, 104, 512] buffer equals mla_post on
    the explicit [R, S, 12, 512] view."""
    m = gpu_lib
    w = synth.dcp8()
    d = device_inputs(w)
    ob = d["o_buf"]  # [256, 104, 512]
    lse_g = torch.from_numpy(w.lse_buf).cuda()  # [256, 96]
    say("ranks helper")
    a = to_bits(m.mla_post_ranks(ob, lse_g, 8, d["w_v"], d["w_v_scale"], d["gate"]))
    b = to_bits(m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"]))
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- the stand-alone quantiser


def test_quantizer_exhaustive(gpu_lib):
    """The device quantiser equals the oracle's on every bf16 pattern (each in
    blocks with different maxima), bit for bit."""
    m = gpu_lib
    say("quantiser exhaustive")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # finite patterns
    rng = np.random.default_rng(30)
    for perm in range(3):
        x = rng.permutation(b) if perm else b.copy()
        pad = (-x.size) % 512
        x = np.concatenate([x, np.zeros(pad, np.uint16)]).reshape(-1, 512)
        codes, scales = m.quantize_mxfp4(bf16_to_dev(x, "cuda"))
        torch.cuda.synchronize()
        rc, rs = O.quantize_mxfp4(x)
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)
    # odd widths and a strided input
    x = O.rne_bf16(rng.standard_normal((37, 96)) * 3.0)
    wide = bf16_to_dev(np.concatenate([x, x], axis=1), "cuda")
    codes, scales = m.quantize_mxfp4(wide[:, :96])
    torch.cuda.synchronize()
    rc, rs = O.quantize_mxfp4(x)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


def every_code_blocks() -> tuple:
    """Blocks of 32 bf16 patterns that meet every E8M0 scale code a finite
    block can have with every element pattern it can hold. For code c, the
    block maximum is fixed to P(c), the largest magnitude pattern whose code
    is c (its exponent c + 2 with a mantissa below 0.75, capped at the largest
    finite value); the other 31 elements run through every finite pattern of
    either sign with magnitude at most P(c), so every (pattern, code) pair a
    block with that code can contain is met. Code 254 would need an infinite
    maximum: the largest finite magnitude 0x7F7F gives code 253."""
    blocks, codes = [], []
    for c in range(1, 254):
        p_hi = min(((c + 3) << 7) - 0x21, 0x7F7F)
        mags = np.arange(0, p_hi + 1, dtype=np.uint32)
        pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-pats.size) % 31
        pats = np.concatenate([pats, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        head = np.full((pats.shape[0], 1), p_hi | (0x8000 if c % 2 else 0), dtype=np.uint16)
        blocks.append(np.concatenate([head, pats], axis=1))
        codes.append(np.full(pats.shape[0], c, dtype=np.uint8))
    return np.concatenate(blocks), np.concatenate(codes)


def test_quantizer_every_scale_code(gpu_lib):
    """The hardware scaled FP4 convert the kernels use (through the
    stand-alone quantiser, which runs the same per-lane code) against the
    oracle's reading of the page's conversion, bit for bit, on every finite
    bf16 pattern under every scale code 1..253 a block of it can get (about
    8.4 million elements)."""
    m = gpu_lib
    blocks, codes = every_code_blocks()
    say(f"quantiser: {blocks.shape[0]} blocks, every scale code")
    pad = (-blocks.shape[0]) % 16
    x = np.concatenate([blocks, np.zeros((pad, 32), np.uint16)]).reshape(-1, 512)
    gc, gs = m.quantize_mxfp4(bf16_to_dev(x, "cuda"))
    torch.cuda.synchronize()
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    assert np.array_equal(gs.reshape(-1)[: codes.size], codes), "scale codes are not the intended ones"
    for r0 in range(0, x.shape[0], 4096):
        rc, rs = O.quantize_mxfp4(x[r0 : r0 + 4096])
        assert np.array_equal(rs, gs[r0 : r0 + 4096]), f"scales differ in rows {r0}.."
        assert np.array_equal(rc, gc[r0 : r0 + 4096]), f"codes differ in rows {r0}.."


def test_quantizer_rows_past_one_grid(gpu_lib):
    """More rows than one pass of the quantiser's capped grid (2^16
    workgroups of 4 rows): every wave strides on, and all 300,000 rows equal
    the oracle's encoding, bit for bit."""
    m = gpu_lib
    say("quantiser 300k rows")
    rng = np.random.default_rng(31)
    x = O.rne_bf16(rng.standard_normal((300000, 32)) * 3.0)
    codes, scales = m.quantize_mxfp4(bf16_to_dev(x, "cuda"))
    torch.cuda.synchronize()
    rc, rs = O.quantize_mxfp4(x)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


def test_quantizer_wv_matches_oracle(gpu_lib):
    """W_V put into MXFP4 on the GPU equals the oracle's encoding."""
    m = gpu_lib
    w = synth.tiny()
    say("quantiser W_V")
    codes, scales = m.quantize_mxfp4(bf16_to_dev(w.wv_bits.reshape(-1, 512), "cuda"))
    torch.cuda.synchronize()
    rc, rs = O.quantize_mxfp4(w.wv_bits)
    assert np.array_equal(codes.cpu().numpy().reshape(rc.shape), rc)
    assert np.array_equal(scales.cpu().numpy().reshape(rs.shape), rs)
