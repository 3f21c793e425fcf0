"""The launch plan (mla_post_plan_for) on the CPU: which kernel, tiling and
grid a call gets, as the host code routes it. mla_post launches exactly this
plan, so these tests pin the routing the GPU tests rely on to reach every
kernel instance, and check that the persistent kernel's schedule covers every
token of every head exactly once."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import mla_split_kv_amd as m


def args(n, S, lse=True):
    """Valid arguments with fake (never dereferenced) device addresses."""
    a = m.MlaPostArgs()
    a.struct_size = ctypes.sizeof(m.MlaPostArgs)
    a.n, a.S = n, S
    a.o = 0x100000
    a.o_sj, a.o_st, a.o_sh = S * 6144, 6144, 512
    if lse:
        a.lse = 0x200000
        a.l_sj, a.l_st, a.l_sh = S * 12, 12, 1
    a.w_v = 0x300000
    a.w_sh, a.w_sv = 128 * 256, 256
    a.w_v_scale = 0x400000
    a.s_sh, a.s_sv, a.s_sb = 128 * 16, 16, 1
    a.gate = 0x500000
    a.core = 0x600000
    return a


def plan(n, S, lse=True, cus=256):
    return m.plan_args(args(n, S, lse), cus)


# (n, S, lse) -> the expected plan at 256 CUs, from the documented rules:
# one-tile instance while one tile per workgroup fits 64 workgroups per head
# and the instance holds every row (8-token tiles up to 3 workgroups per CU,
# i.e. S <= 512, with up to 16 rows; 16-token tiles with up to 8 rows; the
# fewest of 2, 4, 8, 16 rows that hold n); the split-rows kernel for more
# than 16 partials with LSEs up to S = 160 (8-, 4-, 2- or 1-token tiles); else
# the persistent kernel with 64 workgroups per head (40 up to 40 tiles and
# from 65 to 96 tiles, one per tile where that keeps at most 1 or 2 per CU),
# and leftover tokens dealt out evenly from n = 6 (whole 16-token tiles
# below).
TABLE = [
    # the five standard workloads
    ((2, 4, True), dict(kernel="one_tile", tile_tokens=8, rows_held=2, workgroups_per_head=1, workgroups=12)),
    ((1, 64, False), dict(kernel="one_tile", tile_tokens=8, rows_held=1, workgroups_per_head=8, workgroups=96)),
    ((8, 128, True), dict(kernel="one_tile", tile_tokens=8, rows_held=8, workgroups_per_head=16, workgroups=192)),
    ((8, 256, True), dict(kernel="one_tile", tile_tokens=8, rows_held=8, workgroups_per_head=32, workgroups=384)),
    ((16, 4096, True), dict(kernel="persistent", tile_tokens=16, lse_chunks=1, workgroups_per_head=64, workgroups=768,
                            full_tiles=4, short_tokens=0, pair_rows=0)),
    # one-tile boundaries
    ((16, 512, True), dict(kernel="one_tile", tile_tokens=8, rows_held=16, workgroups_per_head=64, workgroups=768)),
    ((8, 513, True), dict(kernel="one_tile", tile_tokens=16, rows_held=8, workgroups_per_head=33)),
    ((4, 1024, True), dict(kernel="one_tile", tile_tokens=16, rows_held=4, workgroups_per_head=64)),
    ((1, 1024, True), dict(kernel="one_tile", tile_tokens=16, rows_held=1, workgroups_per_head=64)),
    ((3, 100, True), dict(kernel="one_tile", tile_tokens=8, rows_held=4)),
    ((5, 100, True), dict(kernel="one_tile", tile_tokens=8, rows_held=8)),
    ((9, 100, True), dict(kernel="one_tile", tile_tokens=8, rows_held=16)),
    ((1, 1000, False), dict(kernel="one_tile", tile_tokens=16, rows_held=1, workgroups_per_head=63)),
    ((16, 513, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=0, short_tokens=13)),
    ((17, 161, True), dict(kernel="persistent", workgroups_per_head=11, full_tiles=0, short_tokens=15)),
    ((1, 1025, False), dict(kernel="persistent", workgroups_per_head=40, pair_rows=0)),
    # both tokens' rows a tile ahead for n <= 4 with LSEs
    ((3, 4096, True), dict(kernel="persistent", workgroups_per_head=64, pair_rows=4)),
    ((4, 2048, True), dict(kernel="persistent", workgroups_per_head=64, pair_rows=4)),
    # two partials with LSEs: the one-tile instance below 6 tokens per CU
    # (S = 1536 at 256 CUs), the streaming kernel from there (8-token tiles,
    # 2 workgroups per CU: 43 for heads 0..7, 42 for heads 8..11, leftover
    # tokens dealt out evenly)
    ((2, 1535, True), dict(kernel="one_tile", tile_tokens=16, rows_held=2, workgroups_per_head=96)),
    ((2, 1536, True), dict(kernel="stream", tile_tokens=8, rows_held=2, workgroups_per_head=43, workgroups=512,
                           full_tiles=4, short_tokens=4)),
    ((2, 8200, True), dict(kernel="stream", tile_tokens=8, rows_held=2, workgroups_per_head=43, full_tiles=23,
                           short_tokens=7)),
    ((2, 1 << 20, True), dict(kernel="stream", tile_tokens=8, workgroups_per_head=43, workgroups=512)),
    # one partial, with an LSE or not, is copied: the one-tile instance while
    # it fits, the persistent kernel up to 6 tokens per CU, then the
    # streaming kernel (16-token tiles)
    ((1, 1535, True), dict(kernel="persistent", workgroups_per_head=40, pair_rows=0)),
    ((1, 1536, True), dict(kernel="stream", tile_tokens=16, rows_held=1, workgroups_per_head=43, full_tiles=2,
                           short_tokens=4)),
    ((1, 4096, True), dict(kernel="stream", tile_tokens=16, rows_held=1, workgroups_per_head=43, full_tiles=5,
                           short_tokens=16)),
    ((1, 4096, False), dict(kernel="stream", tile_tokens=16, rows_held=1)),
    ((1, 1 << 20, True), dict(kernel="stream", workgroups_per_head=43)),
    ((5, 2048, True), dict(kernel="persistent", workgroups_per_head=64, pair_rows=0)),
    # the one-round rule (65 to 96 tiles) and the leftover deal
    ((16, 1100, True), dict(kernel="persistent", workgroups_per_head=40, workgroups=480, full_tiles=1, short_tokens=12)),
    ((4, 1100, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=1, short_tokens=16)),
    ((16, 1536, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=2, short_tokens=7)),
    ((16, 1552, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=1, short_tokens=9)),
    ((16, 4112, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=4, short_tokens=1)),
    ((5, 4112, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=4, short_tokens=16)),
    ((16, 9000, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=8, short_tokens=13)),
    # LSE chunks
    ((64, 400, True), dict(kernel="persistent", lse_chunks=1)),
    ((65, 400, True), dict(kernel="persistent", lse_chunks=2)),
    ((200, 400, True), dict(kernel="persistent", lse_chunks=4)),
    ((512, 400, True), dict(kernel="persistent", lse_chunks=8, workgroups_per_head=40)),
    # between one workgroup per CU and fill tiles: 40 per head up to 40 tiles
    # (one short tile each), one per tile while that is at most 2 per CU (41,
    # 42 tiles), else 64 (a short tile each); one tile each at S = 337 with
    # up to 128 splits (only the 1-token last tile is past the first round)
    ((20, 337, True), dict(kernel="persistent", workgroups_per_head=22, full_tiles=0, short_tokens=16)),
    ((256, 337, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=0, short_tokens=9)),
    ((20, 352, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=0, short_tokens=9)),
    ((32, 640, True), dict(kernel="persistent", workgroups_per_head=40, full_tiles=1, short_tokens=0)),
    ((32, 656, True), dict(kernel="persistent", workgroups_per_head=41, full_tiles=1, short_tokens=0)),
    ((32, 672, True), dict(kernel="persistent", workgroups_per_head=42, full_tiles=1, short_tokens=0)),
    ((32, 688, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=0, short_tokens=11)),
    ((16, 768, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=0, short_tokens=12)),
    ((64, 1024, True), dict(kernel="persistent", workgroups_per_head=64, full_tiles=1, short_tokens=0)),
    # the split-rows kernel: the tile (8, 4, 2 or 1 tokens, at most 8 batches
    # of 16 rows per wave) whose busiest CU has the least to do by the round
    # model; one round: the largest grid within the CUs
    ((17, 64, True), dict(kernel="split_rows", tile_tokens=4, rows_held=16, lse_chunks=1, workgroups_per_head=16,
                          workgroups=192)),
    ((17, 16, True), dict(kernel="split_rows", tile_tokens=1, rows_held=8, workgroups_per_head=16)),
    ((17, 32, True), dict(kernel="split_rows", tile_tokens=2, rows_held=16, workgroups_per_head=16)),
    ((64, 160, True), dict(kernel="split_rows", tile_tokens=8, lse_chunks=1, workgroups_per_head=20, workgroups=240)),
    ((64, 100, True), dict(kernel="split_rows", tile_tokens=8, lse_chunks=1, workgroups_per_head=13)),
    ((65, 100, True), dict(kernel="split_rows", tile_tokens=8, rows_held=16, lse_chunks=2, workgroups_per_head=13)),
    ((128, 7, True), dict(kernel="split_rows", tile_tokens=1, lse_chunks=2, workgroups_per_head=7, workgroups=84)),
    # 129 splits at S = 100: 4-token tiles (the most 4 LSE chunks allow) would
    # put 2 workgroups on some CUs; 2-token tiles, 3 rounds of half the rows, win
    ((129, 100, True), dict(kernel="split_rows", tile_tokens=2, rows_held=16, lse_chunks=4, workgroups=600)),
    ((200, 5, True), dict(kernel="split_rows", tile_tokens=1, lse_chunks=4)),
    ((512, 2, True), dict(kernel="split_rows", tile_tokens=1, rows_held=16, lse_chunks=8, workgroups_per_head=2,
                          workgroups=24)),
    # the split-rows bound: S <= 160 below 64 splits, S <= 192 from 64
    ((63, 161, True), dict(kernel="persistent", workgroups_per_head=11)),
    ((64, 192, True), dict(kernel="split_rows", tile_tokens=4, lse_chunks=1, workgroups_per_head=48)),
    ((512, 193, True), dict(kernel="persistent", lse_chunks=8, workgroups_per_head=13)),
]


@pytest.mark.parametrize("key,expect", TABLE, ids=[f"n{k[0]}_S{k[1]}{'' if k[2] else '_nolse'}" for k, _ in TABLE])
def test_routing_table_at_256_cus(key, expect):
    p = plan(*key)
    assert p["cus"] == 256
    for field, value in expect.items():
        assert p[field] == value, (field, p)
    if p["kernel"] == "one_tile":
        assert p["lse_chunks"] == 1 and p["full_tiles"] == 0 and p["short_tokens"] == 0 and p["pair_rows"] == 0
    elif p["kernel"] == "split_rows":
        assert p["full_tiles"] == 0 and p["short_tokens"] == 0 and p["pair_rows"] == 0
        assert p["workgroups"] == 12 * p["workgroups_per_head"]
    elif p["kernel"] == "stream":
        assert p["tile_tokens"] == 16 // key[0] and p["rows_held"] == key[0] and p["pair_rows"] == 0
        assert p["workgroups"] == 2 * p["cus"] and p["workgroups_per_head"] == -(-p["workgroups"] // 12)
    else:
        assert p["tile_tokens"] == 16 and p["rows_held"] == 0
        assert p["pair_rows"] == (4 if key[2] and 2 <= key[0] <= 4 else 0)


def test_empty_batch_launches_nothing():
    p = plan(4, 0)
    assert p["kernel"] == "none" and p["workgroups"] == 0 and p["cus"] == 256


def test_invalid_arguments_give_the_check_status():
    lib = m.load()
    a = args(4, 8)
    a.o = 0x100001  # misaligned
    out = m.MlaPostPlan()
    assert lib.mla_post_plan_for(ctypes.byref(a), 256, ctypes.byref(out)) == lib.mla_post_check(ctypes.byref(a)) == -3
    assert lib.mla_post_plan_for(ctypes.byref(args(4, 8)), 256, None) == -1


def schedule(S, k, tt):
    """The schedule rule for k workgroups of a head: full tiles of tt tokens
    at stride k, then the leftover tokens dealt out evenly (runs of
    ceil(rest / k)): (full tiles, short tokens)."""
    main = S // (tt * k)
    rest = S - main * tt * k
    return main, -(-rest // k)


def covered(p, S, k=None):
    """Token -> number of persistent or streaming workgroups of one head that
    own it, from the plan's fields and the schedule rule (full tiles at
    stride k, then the leftover tokens in consecutive runs of short_tokens,
    slot by slot). k: a streaming head's own workgroup count, when it differs
    from workgroups_per_head (its tiles then follow the same rule)."""
    k0, main, chunk, tt = p["workgroups_per_head"], p["full_tiles"], p["short_tokens"], p["tile_tokens"]
    if k is None or k == k0:
        k = k0
    else:
        main, chunk = schedule(S, k, tt)
    count = np.zeros(S, dtype=np.int64)
    for slot in range(k):
        for i in range(main):
            t0 = (slot + i * k) * tt
            count[t0 : t0 + tt] += 1
        base = main * tt * k
        t0 = base + slot * chunk
        if chunk and t0 < S:
            count[t0 : min(t0 + chunk, S)] += 1
    return count


@pytest.mark.parametrize("cus", [256, 304, 80, 32])
def test_schedule_covers_every_token_once(cus):
    """Over many (n, S): each token of a head belongs to exactly one workgroup,
    short tiles hold at most 16 tokens, and the grid is 12 per head; the
    one-tile instance's grid covers S."""
    rng = np.random.default_rng(cus)
    sizes = sorted(set([1, 2, 15, 16, 17, 337, 352, 500, 640, 656, 672, 688, 768, 960, 1023, 1024, 1025, 1100, 1536,
                        1537, 2064, 4096, 4112, 9000]
                       + list(rng.integers(1, 20000, size=60))))
    for S in sizes:
        for n, lse in ((1, False), (1, True), (2, True), (4, True), (6, True), (16, True), (20, True), (100, True),
                       (256, True)):
            p = plan(n, int(S), lse, cus)
            assert p["cus"] == cus
            if p["kernel"] == "stream":
                # heads below workgroups mod 12 have workgroups_per_head
                # workgroups, the others one fewer; each head's tokens are
                # covered once either way
                w, k = p["workgroups"], p["workgroups_per_head"]
                assert w == 2 * cus and k == -(-w // 12)
                assert (p["full_tiles"], p["short_tokens"]) == schedule(int(S), k, p["tile_tokens"])
                assert 0 <= p["short_tokens"] <= p["tile_tokens"]
                for kh in {w // 12 + (h < w % 12) for h in range(12)}:
                    assert 0 <= schedule(int(S), kh, p["tile_tokens"])[1] <= p["tile_tokens"]
                    assert np.all(covered(p, int(S), kh) == 1), (n, S, cus, kh, p)
                continue
            assert p["workgroups"] == 12 * p["workgroups_per_head"]
            if p["kernel"] in ("one_tile", "split_rows"):
                assert p["workgroups_per_head"] * p["tile_tokens"] >= S > (p["workgroups_per_head"] - 1) * p["tile_tokens"]
                continue
            assert 0 <= p["short_tokens"] <= p["tile_tokens"]
            c = covered(p, int(S))
            assert np.all(c == 1), (n, S, cus, p)


def split_model(n, S, cus):
    """The tile the documented model picks: tiles of 8, 4, 2, 1 tokens whose
    waves (8 / tile per token) stream at most 8 batches of 16 rows of an
    instance with ceil(n / 64) rounded to 1, 2, 4, 8 LSE chunks; cost =
    ceil(grid / CUs) x (150 + tile x n); the least cost, the larger tile on a
    tie."""
    nch = 1 if n <= 64 else 2 if n <= 128 else 4 if n <= 256 else 8
    best, best_cost = None, None
    for tt in (8, 4, 2, 1):
        g = 8 // tt
        if 64 * nch // g > 16 * 8:
            continue
        cost = -(-12 * -(-S // tt) // cus) * (150 + tt * n)
        if best_cost is None or cost < best_cost:
            best, best_cost = tt, cost
    return best, nch


def test_split_rows_rule():
    """Over n and S at several CU counts: the split-rows kernel exactly when
    n > 16 with LSEs and 16 x 12 x ceil(S / 16) <= 8 CUs (9 CUs from 64
    splits), with the tile and LSE chunks of the model and the rows a wave
    holds at once."""
    for cus in (256, 304, 80, 32):
        for n in (1, 2, 16, 17, 31, 32, 33, 64, 65, 100, 128, 129, 256, 257, 512):
            for S in (1, 2, 3, 5, 16, 22, 31, 32, 33, 43, 63, 64, 86, 100, 144, 160, 161, 176, 192, 193, 250, 336):
                for lse in (True, False):
                    if not lse and n > 1:
                        continue
                    p = plan(n, S, lse, cus)
                    want = lse and n > 16 and 16 * 12 * -(-S // 16) <= (9 if n >= 64 else 8) * cus
                    assert (p["kernel"] == "split_rows") == want, (n, S, cus, p)
                    if not want:
                        continue
                    tt, nch = split_model(n, S, cus)
                    assert (p["tile_tokens"], p["lse_chunks"]) == (tt, nch), (n, S, cus, p)
                    assert p["rows_held"] == min(16, 64 * nch * tt // 8)
                    assert p["workgroups"] == 12 * -(-S // tt)


def test_grid_fits_a_dispatch():
    """Every plan's grid, in work-items (512 per workgroup), fits the 32-bit
    count of a dispatch, up to the largest S the ABI accepts."""
    for S in (1 << 20, (1 << 20) + 1, 1 << 24, 1 << 30):
        for n, lse in ((1, True), (2, True), (3, True), (16, True), (1, False), (512, True)):
            p = plan(n, S, lse)
            assert p["workgroups"] * 512 < 1 << 32, (n, S, p)


def test_current_device_without_gpu_assumes_256():
    """cus = 0 asks the HIP runtime; with no GPU it cannot tell and the plan is
    made for 256 CUs (an MI355X). On a GPU machine the device's own count."""
    p = m.plan_args(args(16, 4096), 0)
    assert p["cus"] > 0
    if p["cus"] == 256:
        assert p == plan(16, 4096)


@pytest.mark.gpu
def test_device_plan_is_the_table(gpu_lib):
    """On the MI355X the current device has 256 CUs, so the plans mla_post
    launches there are the ones the table above pins."""
    for (n, S, lse), _ in TABLE:
        assert m.plan_args(args(n, S, lse), 0) == plan(n, S, lse)


def test_oproj_plan_tiles():
    """o_proj's tile at 256 CUs: 256 x 256 while that grid gives each CU a
    workgroup (the large batch: 16 x 28 tiles), 128 x 128 while that grid
    gives each CU two, smaller tiles for small batches; the grid covers S x
    D."""
    import mla_split_kv_amd as m

    p = m.oproj_plan(4096, 7168, 256)
    assert (p["tile_m"], p["tile_n"], p["workgroups"]) == (256, 256, 16 * 28)
    p = m.oproj_plan(2048, 7168, 256)  # 8 x 28 = 224 large tiles: fewer than the CUs
    assert (p["tile_m"], p["tile_n"], p["workgroups"]) == (128, 128, 16 * 56)
    p = m.oproj_plan(64, 7168, 256)
    assert (p["tile_m"], p["tile_n"]) == (64, 64) and p["workgroups"] == 112
    for S, D in ((1, 8), (37, 136), (300, 1024), (4096, 7168), (5000, 264)):
        p = m.oproj_plan(S, D, 256)
        assert p["workgroups"] == -(-S // p["tile_m"]) * -(-D // p["tile_n"])
