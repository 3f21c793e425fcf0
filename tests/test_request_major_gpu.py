"""Request-major split slices and push-side masking on the GPU, against the
oracle (the mla_back page's combine_splits addressing and stage_push
masking). All through the C ABI."""

from __future__ import annotations

import ctypes
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


def reference(w, d):
    """Oracle inputs for w: the logical per-token partials (what split j of
    token t holds) with the push-side masks applied to the LSEs."""
    o_log, l_log = w.notes["o_logical"], w.notes["lse_logical"]
    lse = O.push_mask(l_log, w.q, w.kv_lens, w.qsl)
    return O.mla_post(o_log, lse, d["w_codes"], d["w_scales"], w.gate)


def check(m, w):
    say(f"{w.name}: per={w.n} q={w.q} S={w.S} o_sr={w.o_sr} masks={w.kv_lens is not None, w.qsl is not None}")
    d = device_inputs(w)
    g = run_debug(m, d)
    ref = reference(w, d)
    st = {}
    st.update(C.check_t1(g["lat"], ref))
    st.update(C.check_t2(g["lat"], g["codes"], g["scales"]))
    st.update(C.check_t3(g["core"], g["codes"], g["scales"], d["w_codes"], d["w_scales"], w.gate))
    st.update(C.check_t4(g["core"], ref, g["lat"], g["codes"], g["scales"]))
    say(f"{w.name}: {st}")
    return g, ref, d


def test_page_dense_layout(gpu_lib):
    """The page's layout: one [P, S, 12, 512] tensor of split slices, token t
    merging slices (t // q) * per + j; every other row is NaN."""
    w = synth.request_major("rm_page", per=4, q=4, S=64, seed=40)
    o_all = np.lib.stride_tricks.as_strided(w.o_buf, shape=w.o_buf.shape)
    og, lg = O.gather_request_major(o_all, w.lse_buf, w.q)
    assert np.array_equal(og, w.notes["o_logical"]) and np.array_equal(lg, w.notes["lse_logical"])
    g, _, _ = check(gpu_lib, w)
    assert np.all(np.isfinite(O.bf16_to_f64(g["core"])))


def test_page_dense_binding_helper(gpu_lib):
    """mla_post_request_major on the whole [P, S, 12, 512] tensor equals the
    explicit strided call."""
    m = gpu_lib
    w = synth.request_major("rm_helper", per=2, q=8, S=48, seed=43)
    d = device_inputs(w)
    base = run_debug(m, d)
    o_all = d["o_buf"]
    lse_all = torch.from_numpy(w.lse_buf).cuda()
    say("request-major helper")
    core = m.mla_post_request_major(o_all, lse_all, w.q, d["w_v"], d["w_v_scale"], d["gate"])
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core), base["core"])


def test_compact_layout_ragged(gpu_lib):
    """Compact request-major [R, per, q, 12, 512]: no unused rows, S = 36 (a
    ragged last tile)."""
    check(gpu_lib, synth.request_major("rm_compact", per=3, q=4, S=36, seed=41, compact=True))


def test_masks(gpu_lib):
    """kv_lens zeros (30% of partial-request pairs) and a batch ending at 33
    of 40 tokens: masked partials count as -inf; tokens past the batch are +0."""
    g, ref, _ = check(gpu_lib, synth.request_major("rm_masked", per=5, q=2, S=40, seed=42, kv_zero=0.3, batch_rows=33))
    assert np.all(g["core"][33:] == 0) and np.all(g["lat"][33:] == 0)


@pytest.mark.parametrize("per,q,S,end,tt", [(24, 2, 128, 120, 8), (40, 4, 40, 34, 2)], ids=["tile8", "tile2"])
def test_split_rows_masks(gpu_lib, per, q, S, end, tt):
    """Many splits per request in the compact layout, with masks, on the
    split-rows kernel: 8-token tiles spanning four requests of q = 2 (one wave
    per token), and 2-token tiles inside requests of q = 4 (four waves per
    token). kv_lens zeros count as -inf and tokens past the batch are +0."""
    m = gpu_lib
    w = synth.request_major(f"rm_split_rows_{tt}", per=per, q=q, S=S, seed=46 + tt, compact=True, kv_zero=0.3,
                            batch_rows=end)
    d = device_inputs(w)
    p = m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], **d["layout"])
    assert p["kernel"] == "split_rows" and p["tile_tokens"] == tt, p
    g, ref, _ = check(m, w)
    assert np.all(g["core"][end:] == 0) and np.all(g["lat"][end:] == 0)


@pytest.mark.parametrize("S", [40, 1104], ids=["one_tile", "persistent"])
def test_one_partial_with_lse_masks(gpu_lib, S):
    """One partial per request with LSEs (copied, not merged) under push-side
    masks: partials of requests with no KV and tokens past the batch give
    +0; every other token meets T1-T4, on both copy routes."""
    m = gpu_lib
    w = synth.request_major(f"rm_copy_S{S}", per=1, q=4, S=S, seed=60 + S % 7, compact=True, kv_zero=0.3,
                            batch_rows=S - 7)
    d = device_inputs(w)
    p = m.plan(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], **d["layout"])
    assert p["kernel"] == ("one_tile" if S == 40 else "persistent"), p
    g, ref, _ = check(m, w)
    assert np.all(g["core"][S - 7:] == 0) and np.all(g["lat"][S - 7:] == 0)
    dead = np.repeat(w.kv_lens[0] == 0, 4)
    assert np.all(g["lat"][dead] == 0)


def test_shared_kv_row_dense_splits(gpu_lib):
    """Dense split partials with one shared row of KV lengths ([S // q]) and
    q = 4: a request with no KV yields +0 for its tokens."""
    m = gpu_lib
    w = synth.dense_splits("shared_kv", 3, 32, seed=44, p_neg_inf=0.1)
    kv = np.array([5, 0, 7, 0, 1, 2, 0, 9], dtype=np.int32)  # R = 8 requests of 4 tokens
    d = device_inputs(w)
    say("shared kv row")
    core, lat, codes, scales = m.mla_post(
        d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], debug=True, q=4, kv_lens=torch.from_numpy(kv).cuda()
    )
    torch.cuda.synchronize()
    lse = O.push_mask(w.lse_view(), 4, np.tile(kv, (3, 1)), None)
    ref = O.mla_post(w.o_view(), lse, d["w_codes"], d["w_scales"], w.gate)
    lat, core = to_bits(lat), to_bits(core)
    C.check_t1(lat, ref)
    C.check_t2(lat, codes.cpu().numpy(), scales.cpu().numpy())
    C.check_t4(core, ref, lat, codes.cpu().numpy(), scales.cpu().numpy())
    dead = np.repeat(kv == 0, 4)
    assert np.all(core[dead] == 0)


def test_no_lse_with_masks(gpu_lib):
    """One partial without LSE: a masked request or a token past the batch
    gives +0; every other token keeps its row bit for bit."""
    m = gpu_lib
    w = synth.single_partial("nolse_masked", 24, seed=45)
    kv = np.array([3, 0, 1, 4, 0, 2], dtype=np.int32)
    qsl = np.array([0, 4, 8, 12, 16, 20, 22], dtype=np.int32)
    d = device_inputs(w)
    say("no-LSE with masks")
    core, lat, codes, scales = m.mla_post(
        d["o"], None, d["w_v"], d["w_v_scale"], d["gate"], debug=True, q=4,
        kv_lens=torch.from_numpy(kv).cuda(), qsl=torch.from_numpy(qsl).cuda(),
    )
    torch.cuda.synchronize()
    lse = O.push_mask(np.zeros((1, 24, 12), np.float32), 4, kv[None, :], qsl)
    ref = O.mla_post(w.o_view(), lse, d["w_codes"], d["w_scales"], w.gate)
    lat = to_bits(lat)
    C.check_t1(lat, ref, exact=True)
    C.check_t4(to_bits(core), ref, strict=True)


def test_version1_struct(gpu_lib):
    """A caller built against the version-1 struct (struct_size 176) gets the
    version-1 behaviour: the later fields are not read."""
    m = gpu_lib
    w = synth.split_merge()
    d = device_inputs(w)
    base = run_debug(m, d)
    core = torch.empty((w.S, 1536), dtype=torch.bfloat16, device="cuda")
    a = m.make_args(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], core)
    a.struct_size = m.ARGS_V1_SIZE
    # junk past the version-1 prefix, chosen so that validation would reject
    # it (q not dividing S, an odd stride, a misaligned pointer) if it were read
    a.q, a.o_sr, a.kv_lens = 7, 3, 0x11
    say("version-1 struct")
    st = m.load().mla_post(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(to_bits(core), base["core"])


def test_large_request_major_full(gpu_lib):
    """Full-size large decode batch in the compact request-major layout
    [1024, 16, 4, 12, 512], launched as the benchmark launches it and with
    stage outputs (core bit-identical); T1-T4 on every one of the 4096
    tokens."""
    m = gpu_lib
    w = synth.large_decode_request_major()
    say(f"{w.name}: per={w.n} q={w.q} S={w.S}")
    d = device_inputs(w)
    core_plain = m.mla_post(d["o"], d["lse"], d["w_v"], d["w_v_scale"], d["gate"], **d["layout"])
    torch.cuda.synchronize()
    g = run_debug(m, d)
    assert np.array_equal(to_bits(core_plain), g["core"])
    o_log, l_log = w.notes["o_logical"], w.notes["lse_logical"]
    st = C.check_all(o_log, l_log, d["w_codes"], d["w_scales"], w.gate, g)
    say(f"{w.name}: all tokens {st}")


@pytest.mark.parametrize(
    "make",
    [
        # 16 splits on 8-token tiles (the one-tile instance holding 16 rows)
        pytest.param(lambda: synth.request_major("rm_masked_n16", per=16, q=4, S=64, seed=46, compact=True,
                                                 kv_zero=0.3, batch_rows=50), id="n16_S64"),
        # 20 splits: the persistent kernel with one tile per workgroup (with
        # fewer tokens, 20 splits take the split-rows kernel)
        pytest.param(lambda: synth.request_major("rm_masked_n20", per=20, q=4, S=400, seed=49, compact=True,
                                                 kv_zero=0.3, batch_rows=350), id="n20_S400"),
        # several tiles per workgroup, the batch ending inside a tile
        pytest.param(lambda: synth.request_major("rm_masked_long", per=16, q=4, S=1104, seed=47, compact=True,
                                                 kv_zero=0.2, batch_rows=1001), id="n16_S1104"),
    ],
)
def test_masks_persistent(gpu_lib, make):
    """Push-side masks with many splits (the persistent kernel, whose LSEs and
    KV lengths are loaded a tile ahead, and the 16-row one-tile instance):
    masked partials count as -inf, tokens past the batch are +0, every token
    checked against the oracle."""
    w = make()
    g, _, _ = check(gpu_lib, w)
    end = int(w.qsl[w.S // w.q])
    assert np.all(g["core"][end:] == 0) and np.all(g["lat"][end:] == 0)


def test_no_lse_masks_persistent(gpu_lib):
    """One partial without LSE at S = 1100 (the persistent kernel): a masked
    request or a token past the batch gives +0, every other token keeps its
    row bit for bit."""
    m = gpu_lib
    S, q = 1100, 4
    R = S // q
    w = synth.single_partial("nolse_masked_long", S, seed=48)
    rng = np.random.default_rng(48)
    kv = rng.integers(0, 4, size=R).astype(np.int32)  # a quarter of the requests have no KV
    qsl = (np.arange(R + 1) * q).astype(np.int32)
    qsl[R] = 1037
    d = device_inputs(w)
    say("no-LSE with masks, persistent")
    core, lat, codes, scales = m.mla_post(
        d["o"], None, d["w_v"], d["w_v_scale"], d["gate"], debug=True, q=q,
        kv_lens=torch.from_numpy(kv).cuda(), qsl=torch.from_numpy(qsl).cuda(),
    )
    torch.cuda.synchronize()
    lse = O.push_mask(np.zeros((1, S, 12), np.float32), q, kv[None, :], qsl)
    ref = O.mla_post(w.o_view(), lse, d["w_codes"], d["w_scales"], w.gate)
    lat = to_bits(lat)
    C.check_t1(lat, ref, exact=True)
    C.check_t4(to_bits(core), ref, strict=True)
    assert np.all(lat[1037:] == 0)
