"""The split-KV decode attention and its fusion with mla_post
(include/mla_decode.h) on the GPU, through the C ABI, against the float64
oracles (oracle/attention.py for the partials, oracle/post.py for the merge
and W_UV).

Each case checks:
  T0     the partials and LSEs the attention leaves in the workspace against
         the attention oracle (criteria.check_t0);
  T1-T4  the fused launch's merge stage outputs and core against the
         mla_post oracle run on those same partials;
  the fused launch's core bit for bit against the unfused pair (the
  attention alone, then mla_post on the workspace's partials in its
  request-major layout), and every counter (the requests' and the unit
  queue's) back at zero after each launch.
The launch has two workgroups per CU, each taking units from a queue once
its first is done; the cases with more (request, split) units than that
(640, 720, 2100 and 5500 at 256 CUs, of ragged lengths) make workgroups
take several. The bench's full size (1024 requests x 4 tokens, 16 splits,
4096 rows each) is checked on eight sampled requests against the oracles
and on the whole core against the unfused pair.
Inputs are seeded and synthetic (synth.decode_inputs).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import criteria as C
import oracle.attention as A
import oracle.post as O
import synth
from gpu_support import bf16_to_dev, to_bits

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def device_case(d, qry_pad=0, kv_pad=0):
    """Device tensors of DecodeInputs d; queries and cache rows optionally as
    views of wider buffers (row strides 576 + pad)."""
    dev = "cuda"
    if qry_pad:
        wide = torch.zeros((d.S, 12, 576 + qry_pad), dtype=torch.bfloat16, device=dev)
        wide[:, :, :576] = bf16_to_dev(d.qry, dev)
        qry = wide[:, :, :576]
    else:
        qry = bf16_to_dev(d.qry, dev)
    if kv_pad:
        wide = torch.zeros((max(1, d.kv.shape[0]), 576 + kv_pad), dtype=torch.bfloat16, device=dev)
        if d.kv.shape[0]:
            wide[: d.kv.shape[0], :576] = bf16_to_dev(d.kv, dev)
        kv = wide[: max(1, d.kv.shape[0]), :576]
    else:
        kv = bf16_to_dev(d.kv if d.kv.shape[0] else np.zeros((1, 576), np.uint16), dev)
    wc, ws = O.quantize_mxfp4(d.wv_bits)
    return {
        "qry": qry,
        "kv": kv,
        "indptr": torch.from_numpy(d.indptr).to(dev),
        "w_v": torch.from_numpy(wc).to(dev),
        "w_s": torch.from_numpy(ws).to(dev),
        "gate": bf16_to_dev(d.gate, dev),
        "wc": wc,
        "ws": ws,
    }


def check_case(m, d, **pads):
    say(f"{d.name}: R={d.R} q={d.q} n={d.n} lens={np.diff(d.indptr).tolist()[:8]}.. pads={pads}")
    t = device_case(d, **pads)
    ws = m.DecodeWorkspace(d.R, d.q, d.n)
    args = (t["qry"], t["kv"], t["indptr"], d.q, d.n, d.scale, t["w_v"], t["w_s"], t["gate"], ws)
    core, lat, codes, scales = m.mla_decode(*args, debug=True)
    torch.cuda.synchronize()
    cnt = ws.counters().cpu().numpy()
    assert np.all(cnt == 0), f"counters not reset: {cnt[cnt != 0][:8]}"
    po, pl = ws.partials()
    po_h, pl_h = to_bits(po), pl.cpu().numpy()
    g = {"core": to_bits(core), "lat": to_bits(lat), "codes": codes.cpu().numpy(), "scales": scales.cpu().numpy()}
    # the producer against the attention oracle
    ref = A.attention_partials(d.qry, d.kv, d.indptr, d.q, d.n, d.scale)
    lens = np.diff(d.indptr.astype(np.int64))
    nrows = np.stack([np.diff(A.split_bounds(int(L), d.n)) for L in lens]) if d.R else np.zeros((0, d.n))
    st = C.check_t0(po_h, pl_h, ref, nrows)
    # the merge stage against the mla_post oracle on the GPU's own partials
    o_tok = np.ascontiguousarray(np.transpose(po_h, (1, 0, 2, 3, 4)).reshape(d.n, d.S, 12, 512))
    l_tok = np.ascontiguousarray(np.transpose(pl_h, (1, 0, 2, 3)).reshape(d.n, d.S, 12))
    st.update(C.check_all(o_tok, l_tok, t["wc"], t["ws"], d.gate, g))
    # the unfused pair gives the same core, bit for bit
    ws2 = m.DecodeWorkspace(d.R, d.q, d.n)
    m.mla_decode(*args[:-1], ws2, fused=False)
    torch.cuda.synchronize()
    cnt = ws2.counters().cpu().numpy()
    assert np.all(cnt == 0), f"counters not reset by the attention alone: {cnt[cnt != 0][:8]}"
    ov, lv, lay = ws2.token_views()
    core2 = m.mla_post(ov, lv, t["w_v"], t["w_s"], t["gate"], **lay)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(ws2.partials()[0]), po_h), "the attention alone wrote other partials"
    assert np.array_equal(to_bits(core2), g["core"]), "fused and unfused core differ"
    # a second fused call on the same workspace: the same core
    core3 = m.mla_decode(*args)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core3), g["core"]), "a second call on the workspace differs"
    say(f"{d.name}: {st}")
    return st, g, ref


CASES = [
    # (name, lens, q, n, seed, options)
    ("one_request", [200], 4, 3, 1, {}),
    ("ragged_blocks", [1, 63, 64, 65, 129, 300, 0, 17], 4, 4, 2, {}),
    ("empty_splits", [2, 5, 0, 3], 2, 6, 3, {}),  # L < n: some splits empty, one request empty
    ("q1", [100, 37, 250], 1, 5, 4, {}),
    ("q3", [77, 90, 16, 140, 5], 3, 2, 5, {}),
    ("one_split", [130, 66], 4, 1, 6, {}),
    ("many_splits", [700, 500], 4, 64, 7, {}),
    ("R_not_multiple_of_8", [40] * 13, 4, 3, 8, {}),
    ("strided", [90, 33, 160], 4, 3, 9, {"qry_pad": 64, "kv_pad": 32}),
    ("wide_scores", [120, 64], 4, 2, 10, {"q_sigma": 4.0}),
    # more units than workgroups: each workgroup takes several from the queue
    ("many_units", [int(x) for x in np.random.default_rng(11).integers(0, 150, 160)], 4, 4, 11, {}),
    ("many_units_q1", [int(x) for x in np.random.default_rng(12).integers(1, 400, 90)], 1, 8, 12, {}),
    # many requests with ragged lengths, some empty
    ("ragged_300", [int(x) for x in np.random.default_rng(13).integers(0, 200, 300)], 4, 7, 13, {}),
    # more requests than four per CU
    ("requests_1100", [int(x) for x in np.random.default_rng(14).integers(0, 90, 1100)], 2, 5, 14, {}),
]


@pytest.mark.parametrize("name,lens,q,n,seed,opts", CASES, ids=[c[0] for c in CASES])
def test_decode(gpu_lib, name, lens, q, n, seed, opts):
    opts = dict(opts)
    pads = {k: opts.pop(k) for k in ("qry_pad", "kv_pad") if k in opts}
    d = synth.decode_inputs(name, lens, q, n, seed, **opts)
    st, g, _ = check_case(gpu_lib, d, **pads)
    # a request without KV rows: its tokens' core rows are exactly +0
    lens = np.asarray(lens)
    for r in np.nonzero(lens == 0)[0]:
        assert np.all(g["core"][r * q : (r + 1) * q] == 0)


def test_decode_empty_batch_and_errors(gpu_lib):
    m = gpu_lib
    say("decode: R = 0 and argument errors")
    ws = m.DecodeWorkspace(0, 4, 2)
    qry = torch.zeros((0, 12, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 576), dtype=torch.bfloat16, device="cuda")
    indptr = torch.zeros(1, dtype=torch.int32, device="cuda")
    w_v = torch.zeros((12, 128, 256), dtype=torch.uint8, device="cuda")
    w_s = torch.full((12, 128, 16), 127, dtype=torch.uint8, device="cuda")
    gate = torch.zeros((0, 1536), dtype=torch.bfloat16, device="cuda")
    core = m.mla_decode(qry, kv, indptr, 4, 2, 0.1, w_v, w_s, gate, ws)
    torch.cuda.synchronize()
    assert core.shape == (0, 1536)
    with pytest.raises(m.MlaPostError):  # q past MLA_DECODE_QMAX
        m.DecodeWorkspace(1, 5, 2)
    with pytest.raises(m.MlaPostError):  # n past MLA_DECODE_NMAX
        m.DecodeWorkspace(1, 4, 65)


# Seeded random configurations: request counts on both sides of one unit
# per CU pair (512 at 256 CUs), one to four tokens, 1 to 64 splits, ragged
# lengths with empty requests and splits shorter than a block, strided
# queries and cache rows, wide score spreads. Each case runs the whole
# check_case (T0 on the partials, T1-T4 on every token, fused == unfused bit
# for bit, counters back at zero) and is named before it runs.
RANDOM_CASES = 16
MAX_KV_ROWS = 50_000  # total cache rows of a case: the oracle's attention stays in seconds


def random_case(i):
    rng = np.random.default_rng(7000 + i)
    R = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 512)), int(rng.integers(512, 900))]))
    q = int(rng.integers(1, 5))
    n = int(rng.choice([1, 2, 3, int(rng.integers(4, 17)), int(rng.integers(17, 65))]))
    mean = max(1, MAX_KV_ROWS // R)
    lens = rng.integers(0, 2 * mean + 1, R)
    lens[rng.random(R) < 0.1] = 0
    short = rng.random(R) < 0.1
    lens[short] = rng.integers(1, n + 1, int(short.sum()))  # splits of 0 or 1 rows
    opts = {}
    if rng.random() < 0.3:
        opts["q_sigma"] = float(rng.choice([3.0, 6.0]))
    pads = {}
    if rng.random() < 0.3:
        pads = {"qry_pad": int(rng.choice([8, 64])), "kv_pad": int(rng.choice([8, 32]))}
    return f"rand{i}", [int(x) for x in lens], q, n, 8000 + i, opts, pads


@pytest.mark.parametrize("i", range(RANDOM_CASES))
def test_decode_random(gpu_lib, i):
    name, lens, q, n, seed, opts, pads = random_case(i)
    say(f"random decode case {i}: R={len(lens)} q={q} n={n} rows={sum(lens)} opts={opts} pads={pads}")
    d = synth.decode_inputs(name, lens, q, n, seed, **opts)
    st, g, _ = check_case(gpu_lib, d, **pads)
    lens = np.asarray(lens)
    for r in np.nonzero(lens == 0)[0]:
        assert np.all(g["core"][r * q : (r + 1) * q] == 0)


FULL_R, FULL_Q, FULL_N, FULL_L = 1024, 4, 16, 4096


def test_decode_full_size_sampled(gpu_lib):
    """The bench's decode workload at full size: 1024 requests of 4 tokens, 16
    splits, 4096 cache rows of 576 bf16 each (4.83 GB of KV), in the launch
    the bench times (two persistent workgroups per CU). The oracles check
    eight requests (both ends, around the middle, three seeded picks): their
    partials against the attention oracle (T0), their tokens' merge stage and
    core against the mla_post oracle (T1-T4). The whole core is checked bit
    for bit against the unfused pair and against the same launch without
    stage outputs, and every counter is back at zero."""
    m = gpu_lib
    R, q, n, L = FULL_R, FULL_Q, FULL_N, FULL_L
    say(f"full size: R={R} q={q} n={n} L={L}: drawing the inputs")
    d = synth.decode_inputs("decode_full_size", [L] * R, q, n, 9001)
    t = device_case(d)
    ws = m.DecodeWorkspace(R, q, n)
    args = (t["qry"], t["kv"], t["indptr"], q, n, d.scale, t["w_v"], t["w_s"], t["gate"], ws)
    say("full size: fused launch with stage outputs")
    core, lat, codes, scales = m.mla_decode(*args, debug=True)
    torch.cuda.synchronize()
    cnt = ws.counters().cpu().numpy()
    assert np.all(cnt == 0), f"counters not reset: {cnt[cnt != 0][:8]}"
    core_h = to_bits(core)
    po, pl = ws.partials()
    rng = np.random.default_rng(9002)
    pick = sorted({0, 1, R // 2 - 1, R // 2, R - 1} | {int(x) for x in rng.integers(0, R, 3)})
    nrows = np.diff(A.split_bounds(L, n))[None]
    for r in pick:
        toks = slice(r * q, (r + 1) * q)
        po_h, pl_h = to_bits(po[r : r + 1]), pl[r : r + 1].cpu().numpy()
        ref = A.attention_partials(d.qry[toks], d.kv[r * L : (r + 1) * L], np.array([0, L], np.int32), q, n, d.scale)
        st = C.check_t0(po_h, pl_h, ref, nrows)
        o_tok = np.ascontiguousarray(np.transpose(po_h, (1, 0, 2, 3, 4)).reshape(n, q, 12, 512))
        l_tok = np.ascontiguousarray(np.transpose(pl_h, (1, 0, 2, 3)).reshape(n, q, 12))
        g = {"core": core_h[toks], "lat": to_bits(lat[toks]), "codes": codes[toks].cpu().numpy(),
             "scales": scales[toks].cpu().numpy()}
        st.update(C.check_all(o_tok, l_tok, t["wc"], t["ws"], d.gate[toks], g))
        say(f"full size: request {r}: {st}")
    # the launch the bench times (no stage outputs): the same core
    core_b = m.mla_decode(*args)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(core_b), core_h), "the launch without stage outputs gives another core"
    del lat, codes, scales, core_b
    # the unfused pair: the same core, bit for bit
    ws2 = m.DecodeWorkspace(R, q, n)
    m.mla_decode(*args[:-1], ws2, fused=False)
    ov, lv, lay = ws2.token_views()
    core2 = m.mla_post(ov, lv, t["w_v"], t["w_s"], t["gate"], **lay)
    torch.cuda.synchronize()
    cnt = ws2.counters().cpu().numpy()
    assert np.all(cnt == 0), f"counters not reset by the attention alone: {cnt[cnt != 0][:8]}"
    assert np.array_equal(to_bits(core2), core_h), "fused and unfused core differ"
    say(f"full size: {len(pick)} requests checked against the oracles, core equal to the unfused pair")
    del ws, ws2, core, core2, po, pl, ov, lv, t
    torch.cuda.empty_cache()
