#!/usr/bin/env python3
"""Benchmark of mla_post on one MI355X.

A step is one mla_post call over one batch: the whole path (LSE merge of the
bf16 partial rows, bf16 latents, MXFP4, FP4-MFMA W_UV, gate) in the fused
kernel, with every input already resident in HBM. The workload is the large
decode batch: S = 4096 tokens (1024 requests x 4), 16 KV splits per request,
12 heads, latent 512, o ~ N(0, 2) bf16 [16, 4096, 12, 512] (805 MB),
lse ~ N(8, 6) with 5% -inf, W_V ~ N(0, 1/sqrt(512)) put into MXFP4 by the
library's quantiser, gate ~ U(0, 1) bf16. Inputs are seeded and synthetic.

Prints one JSON line: tokens/s (whole job), ms per step, the roofline of the
fused kernel (algorithmic HBM bytes per launch / its average duration from HIP
events over the timed region, against 8 TB/s) and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --calibrate-copy   # a plain 1 GiB device copy, for counter scaling
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
CSRC = os.path.join(ROOT, "mla_split_kv_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "mla_post.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_hbm_per_launch.json")
# Launches whose HBM traffic comes from committed counter runs: the entry's
# name -> (a substring of the kernel's name in the counter CSVs, its source
# file, what was measured).
TRAFFIC_KERNELS = {
    "large_decode": ("mla_post_kernel", "mla_post.hip", "mla_post_kernel<false, 1, 0> (large_decode workload)"),
    "large_decode_request_major": (
        "mla_post_kernel", "mla_post.hip", "mla_post_kernel<false, 1, 0> (large_decode_request_major workload)"),
    "decode_attention": (
        "mla_decode_kernel<false>", "decode.hip",
        "mla_decode_kernel<false>: the attention alone, 1024 requests x 4 tokens, 16 splits, 4096 rows each"),
    "decode_fused": (
        "mla_decode_kernel<true>", "decode.hip",
        "mla_decode_kernel<true>: attention and mla_post in one launch, same sizes"),
    "oproj": ("oproj_big_kernel", "oproj.hip", "oproj_big_kernel: core [4096, 1536] x W_O [7168, 1536]^T"),
}
W_V_BYTES = 12 * 128 * 256 + 12 * 128 * 16  # MXFP4 codes + E8M0 scales, read once per launch


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_sha(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def live_rows(w) -> int:
    """Partial rows that carry weight, counted from the workload's LSEs: a row
    is live when its LSE is a finite number (NaN and +inf count as -inf);
    every row is live when there are no LSEs."""
    import numpy as np

    if w.lse_buf is None:
        return w.n * w.S * 12
    v = w.notes["lse_logical"] if "lse_logical" in w.notes else w.lse_view()
    return int(np.isfinite(v).sum())


def algorithmic_bytes(w) -> dict:
    """Bytes the method must move per call: each partial row of non-zero
    weight (1 KiB; rows whose LSE is -inf, NaN or +inf need not be read), every
    LSE (4 B), W_V once, the gate read and the core write (S x 1536 bf16 each)."""
    live = live_rows(w)
    n_lse = 0 if w.lse_buf is None else w.n * w.S * 12
    gate_core = 2 * w.S * 1536 * 2
    live_b = live * 1024 + n_lse * 4 + W_V_BYTES + gate_core
    nominal_b = w.n * w.S * 12 * 1024 + n_lse * 4 + W_V_BYTES + gate_core
    return {"live_rows": live, "rows": w.n * w.S * 12, "alg_bytes": live_b, "nominal_bytes": nominal_b}


def device_setup(w, m, torch):
    """Move a workload to the GPU; W_V goes to MXFP4 with the library's quantiser."""
    import numpy as np

    dev = torch.device("cuda", 0)
    o_buf = torch.from_numpy(w.o_buf.view(np.int16)).view(torch.bfloat16).to(dev)
    o = torch.as_strided(o_buf, (w.n, w.S, 12, 512), tuple(w.o_strides) + (1,))
    lse = None
    if w.lse_buf is not None:
        lse = torch.as_strided(torch.from_numpy(w.lse_buf).to(dev), (w.n, w.S, 12), tuple(w.lse_strides))
    wv = torch.from_numpy(w.wv_bits.reshape(-1, 512).view(np.int16)).view(torch.bfloat16).to(dev)
    codes, scales = m.quantize_mxfp4(wv)
    w_v = codes.view(12, 128, 256)
    w_s = scales.view(12, 128, 16)
    gate = torch.from_numpy(w.gate.view(np.int16)).view(torch.bfloat16).to(dev)
    core = torch.empty((w.S, 1536), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, w_v=w_v, w_s=w_s, gate=gate, core=core, o_buf=o_buf)


def layout_args(w) -> dict:
    """Request-major arguments of a workload (none for the dense layouts)."""
    if w.q == 1 and not w.o_sr and not w.l_sr:
        return {}
    return {"q": w.q, "o_sr": w.o_sr, "l_sr": w.l_sr}


def time_gpu(call, steps: int, warmup: int, torch) -> dict:
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"wall_s": wall, "event_ms": ev0.elapsed_time(ev1)}


def time_per_call(call, calls: int, torch, scratch=None) -> float:
    """Median of HIP events around each single call (device synchronised
    between calls). With `scratch` (a 1 GiB device tensor) the calls are cold:
    the scratch is overwritten before each one, so the caches (L2, MALL) hold
    none of the call's inputs; only the call itself is inside the events."""
    import statistics

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(calls):
        if scratch is not None:
            scratch.fill_(1)
        ev0.record()
        call()
        ev1.record()
        torch.cuda.synchronize()
        out.append(1e3 * ev0.elapsed_time(ev1))
    return statistics.median(out)


def time_graph(call, torch, per_graph: int = 100, replays: int = 20) -> float:
    """Microseconds per call when `per_graph` calls are captured in one HIP
    graph and the graph is replayed back to back (no host launch per call).
    The library records no memset in a capture; each replay is checked by the
    graph tests, not here."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(replays):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return 1e3 * ev0.elapsed_time(ev1) / (replays * per_graph)


def copy_ceiling(torch) -> float:
    """Device copy rate (GB/s, bytes read + bytes written) of a plain 1 GiB
    copy: the stream-copy ceiling the kernel is also compared with."""
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t = time_gpu(lambda: dst.copy_(src), 20, 3, torch)
    return 2 * 2 * n * 20 / (t["event_ms"] * 1e-3) / 1e9


def cpu_baseline(w, tokens: int) -> dict:
    """The oracle as it is, single-threaded (BLAS limited to one thread), on
    the first `tokens` tokens of the same workload; W_V encoded by the
    oracle's own quantiser (not timed)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.post as O

    codes, scales = O.quantize_mxfp4(w.wv_bits)
    if "o_logical" in w.notes:
        o, lse = w.notes["o_logical"], w.notes["lse_logical"]
    else:
        o, lse = w.o_view(), w.lse_view()
    chunk = 64
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for s0 in range(0, tokens, chunk):
            O.mla_post(o, lse, codes, scales, w.gate, tokens=np.arange(s0, min(tokens, s0 + chunk)))
        dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(tokens / dt, 2),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {tokens} of {w.S} tokens of the same workload, in chunks of {chunk}, one thread "
        f"({dt:.1f} s; host {cpu}, {os.cpu_count()} logical CPUs)",
    }


_POOL_STATE = {}


def _pool_init() -> None:
    from threadpoolctl import threadpool_limits

    _POOL_STATE["limit"] = threadpool_limits(limits=1)


def _pool_chunk(bounds) -> int:
    import numpy as np

    import oracle.post as O

    st = _POOL_STATE
    s0, s1 = bounds
    O.mla_post(st["o"], st["lse"], st["codes"], st["scales"], st["gate"], tokens=np.arange(s0, s1))
    return s1 - s0


def cpu_baseline_all_cores(w, tokens: int, workers: int) -> dict:
    """The same oracle calls as cpu_baseline, spread over `workers` forked
    processes (one BLAS thread each) by chunks of 64 tokens. Run before the
    process touches the GPU, so the forked workers inherit no device state."""
    import multiprocessing as mp

    import oracle.post as O

    codes, scales = O.quantize_mxfp4(w.wv_bits)
    if "o_logical" in w.notes:
        o, lse = w.notes["o_logical"], w.notes["lse_logical"]
    else:
        o, lse = w.o_view(), w.lse_view()
    _POOL_STATE.update(o=o, lse=lse, codes=codes, scales=scales, gate=w.gate)
    chunks = [(s0, min(tokens, s0 + 64)) for s0 in range(0, tokens, 64)]
    with mp.get_context("fork").Pool(workers, initializer=_pool_init) as pool:
        pool.map(_pool_chunk, chunks[:workers], chunksize=1)  # workers up, imports done (not timed)
        t0 = time.perf_counter()
        done = sum(pool.map(_pool_chunk, chunks, chunksize=1))
        dt = time.perf_counter() - t0
    _POOL_STATE.clear()
    return {
        "value": round(done / dt, 2),
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"first {tokens} of {w.S} tokens, chunks of 64 over {workers} processes ({dt:.2f} s)",
    }


def traffic_entry(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on this workload (a TRAFFIC_KERNELS entry) and on the current source
    of its kernel."""
    if not os.path.exists(TRAFFIC_FILE) or workload not in TRAFFIC_KERNELS:
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f).get(workload)
    src = os.path.join(CSRC, TRAFFIC_KERNELS[workload][1])
    if not t or t.get("workload") != workload or t.get("kernel_source_sha256") != kernel_sha(src):
        return None
    return t.get("hbm_bytes_per_launch")


def counter_kib(csv_path: str, kernel_substr: str) -> list:
    """Per-dispatch values (KiB) of the one counter in a rocprofv3 --pmc CSV,
    for dispatches whose kernel name contains kernel_substr."""
    import csv

    with open(csv_path) as f:
        return [float(r["Counter_Value"]) for r in csv.DictReader(f) if kernel_substr in r["Kernel_Name"]]


def traffic_from(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                 workload: str = "large_decode") -> dict:
    """HBM bytes per launch of a TRAFFIC_KERNELS entry's kernel from FETCH_SIZE
    / WRITE_SIZE runs (median over its dispatches), each scaled by what the same
    counter reads for the plain 1 GiB copy (true bytes / counter bytes).
    Stored under the entry's name in TRAFFIC_FILE."""
    import statistics

    sub, src, what = TRAFFIC_KERNELS[workload]
    copy_bytes = 1 << 30
    fk = statistics.median(counter_kib(fetch_csv, sub))
    wk = statistics.median(counter_kib(write_csv, sub))
    cf = statistics.median(counter_kib(copy_fetch_csv, "copyBuffer"))
    cw = statistics.median(counter_kib(copy_write_csv, "copyBuffer"))
    f_scale = copy_bytes / (cf * 1024)
    w_scale = copy_bytes / (cw * 1024)
    fetch = fk * 1024 * f_scale
    write = wk * 1024 * w_scale
    out = {
        "kernel": what,
        "workload": workload,
        "kernel_source_sha256": kernel_sha(os.path.join(CSRC, src)),
        "fetch_kib_per_dispatch": fk,
        "write_kib_per_dispatch": wk,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_fetch_bytes": round(fetch),
        "hbm_write_bytes": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
    }
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    table[workload] = out
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    return out


def size_sweep(sizes: list, steps: int, warmup: int, m, torch, splits: int = 16, no_lse: bool = False) -> dict:
    """Microseconds per call and the roofline fraction at several batch sizes
    S, with the large decode batch's distributions (16 splits unless given,
    o ~ N(0, 2), lse ~ N(8, 6) with 5% -inf, seed 4), generated once at the
    largest size; each size takes the first S tokens of it (strided views, as
    a caller would pass them). no_lse: one partial without LSEs instead (o ~
    N(0, 1), seed 3). Beside each: a plain streaming read of as many bytes
    (mla_measure_read), and read_frac = its time over the call's."""
    import numpy as np

    import synth

    smax = max(sizes)
    if no_lse:
        splits = 1
        log(f"generating one partial without LSEs x {smax} tokens")
        w = synth.single_partial(f"sweep_nolse_S{smax}", smax, seed=3)
    else:
        log(f"generating {splits} splits x {smax} tokens ({splits * smax * 12 * 1024 / 1e6:.0f} MB of partials)")
        w = synth.dense_splits(f"sweep_n{splits}_S{smax}", splits, smax, seed=4, o_sigma=2.0, lse_normal=(8.0, 6.0),
                               p_neg_inf=0.05)
    d = device_setup(w, m, torch)
    lse_bytes = 0 if no_lse else splits * 12 * 4
    live_by_token = (np.full(smax, 12) if no_lse else np.isfinite(w.lse_view()).sum(axis=(0, 2)))
    # the plain-read reference of each size: one streaming read of as many
    # bytes as the call's algorithmic bytes, from a buffer of its own
    alg_max = int(live_by_token.sum()) * 1024 + smax * lse_bytes + W_V_BYTES + 2 * smax * 1536 * 2
    rbuf = torch.empty((alg_max + 15) // 16 * 16, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16, dtype=torch.uint8, device="cuda")
    rows = []
    for S in sizes:
        lse = None if no_lse else d["lse"][:, :S]
        call = m.prepare(d["o"][:, :S], lse, d["w_v"], d["w_s"], d["gate"][:S], d["core"][:S])
        t = time_gpu(call, steps, warmup, torch)
        us = 1e3 * t["event_ms"] / steps
        alg = int(live_by_token[:S].sum()) * 1024 + S * lse_bytes + W_V_BYTES + 2 * S * 1536 * 2
        gbps = alg / (us * 1e-6) / 1e9
        nread = (alg + 15) // 16 * 16
        tr = time_gpu(lambda: m.measure_read(rbuf[:nread], sink), steps, warmup, torch)
        read_us = 1e3 * tr["event_ms"] / steps
        rows.append({"S": S, "us_per_call": round(us, 3), "GBps": round(gbps, 1),
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "tokens_per_s": round(S / (us * 1e-6), 1),
                     "alg_bytes": alg, "read_us": round(read_us, 3), "read_frac": round(read_us / us, 4),
                     "plan": m.plan(d["o"][:, :S], lse, d["w_v"], d["w_s"], d["gate"][:S])})
        log(f"S={S}: {rows[-1]}")
    what = "one partial without LSEs" if no_lse else f"{splits} splits, large decode distributions"
    return {"size_sweep": rows, "workload": f"{what}, first S tokens", "steps": steps}


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD's published figure


def oproj_bench(core, D: int, steps: int, warmup: int, m, torch) -> dict:
    """o_proj (include/mla_oproj.h) on the call's own core [S, 1536] with a
    seeded W_O ~ N(0, 1/sqrt(1536)) bf16 [D, 1536]: microseconds per call
    from HIP events, TFLOP/s against the bf16 matrix-core peak, and torch's
    own bf16 matrix product (the vendor BLAS) on the same operands, timed
    the same way, for context."""
    import numpy as np

    import synth

    S, K = int(core.shape[0]), int(core.shape[1])
    rng = np.random.default_rng(99)
    wo_bits = synth.f32_to_bf16_bits(rng.standard_normal((D, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    w_o = torch.from_numpy(wo_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((S, D), dtype=torch.bfloat16, device="cuda")
    call = m.PreparedOproj(core, w_o, out)
    t = time_gpu(call, steps, warmup, torch)
    us = 1e3 * t["event_ms"] / steps
    flops = 2.0 * S * D * K
    tflops = flops / (us * 1e-6) / 1e12
    w_t = w_o.t().contiguous()  # [K, D]: a plain 2-D product of contiguous operands
    ref_out = torch.empty_like(out)
    tb = time_gpu(lambda: torch.mm(core, w_t, out=ref_out), steps, warmup, torch)
    us_blas = 1e3 * tb["event_ms"] / steps
    byts = (S * K + D * K + S * D) * 2
    return {
        "workload": f"core [{S}, {K}] (the call's own) x W_O [{D}, {K}]^T -> bf16 [{S}, {D}]",
        "us_per_call": round(us, 3),
        "tflops": round(tflops, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_entry("oproj") if (S, D, K) == (4096, 7168, 1536) else None},
        "hbm_bytes_min": byts,
        "vendor_blas_us": round(us_blas, 3),
        "vs_vendor_blas": round(us_blas / us, 3),
        "plan": m.oproj_plan(S, D),
    }


def read_ceiling(buf, steps: int, torch, m) -> dict:
    """The plain-read reference (include/mla_measure.h): one streaming read of
    the same partial buffer the fused kernel reads, 16-byte non-temporal loads
    from every CU, timed like the kernel."""
    sink = torch.empty(16, dtype=torch.uint8, device=buf.device)
    t = time_gpu(lambda: m.measure_read(buf, sink), steps, 5, torch)
    us = 1e3 * t["event_ms"] / steps
    n = buf.numel() * buf.element_size()
    return {"us": round(us, 3), "GBps": round(n / (us * 1e-6) / 1e9, 1), "bytes": n}


def decode_bench(R: int, q: int, n: int, L: int, steps: int, warmup: int, m, torch) -> dict:
    """The split-KV decode attention fused with mla_post (include/mla_decode.h)
    at the large decode batch's sizes: R requests of q tokens, n splits, L
    cache rows per request; queries and cache rows ~ N(0, 1) bf16, W_V ~
    N(0, 1/sqrt(512)) into MXFP4 by the library's quantiser, gate ~ U(0, 1),
    drawn on the device from a seeded generator. Times the fused launch, the
    attention alone, mla_post on its partials, and that unfused pair."""
    g = torch.Generator(device="cuda").manual_seed(7)
    S = R * q
    qry = torch.randn((S, 12, 576), generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn((R * L, 576), generator=g, device="cuda").to(torch.bfloat16)
    indptr = torch.arange(R + 1, device="cuda", dtype=torch.int32) * L
    wv = (torch.randn((12 * 128, 512), generator=g, device="cuda") / 512**0.5).to(torch.bfloat16)
    codes, scales = m.quantize_mxfp4(wv)
    w_v, w_s = codes.view(12, 128, 256), scales.view(12, 128, 16)
    gate = torch.rand((S, 1536), generator=g, device="cuda").to(torch.bfloat16)
    core = torch.empty((S, 1536), dtype=torch.bfloat16, device="cuda")
    core2 = torch.empty_like(core)
    ws = m.DecodeWorkspace(R, q, n)
    scale = 1.0 / 192**0.5
    fused = m.PreparedDecode(qry, kv, indptr, q, n, scale, w_v, w_s, gate, ws, core, fused=True)
    attn = m.PreparedDecode(qry, kv, indptr, q, n, scale, w_v, w_s, gate, ws, core, fused=False)
    ov, lv, lay = ws.token_views()
    post = m.prepare(ov, lv, w_v, w_s, gate, core2, **lay)

    def pair():
        attn()
        post()

    # about half a second of fused calls first, so that the timed calls do
    # not start from the clocks and caches of the input generation
    t0 = time.time()
    while time.time() - t0 < 0.5:
        fused()
        torch.cuda.synchronize()
    res = {}
    for name, call in (("fused", fused), ("attention", attn), ("mla_post", post), ("pair", pair)):
        t = time_gpu(call, steps, warmup, torch)
        res[name] = 1e3 * t["event_ms"] / steps
    torch.cuda.synchronize()
    same = bool(torch.equal(core, core2))
    alg = R * L * 1152 + S * 12 * 576 * 2 + W_V_BYTES + 2 * S * 1536 * 2
    measured = (R, q, n, L) == (1024, 4, 16, 4096)  # the sizes of the committed counter runs
    gbps = alg / (res["fused"] * 1e-6) / 1e9
    out = {
        "workload": f"{R} requests x {q} tokens, {n} KV splits, {L} cache rows of 576 bf16 per request, 12 heads",
        "us_fused": round(res["fused"], 1),
        "us_attention_alone": round(res["attention"], 1),
        "us_mla_post_on_partials": round(res["mla_post"], 1),
        "us_unfused_pair": round(res["pair"], 1),
        "fused_vs_pair": round(res["pair"] / res["fused"], 3),
        "tokens_per_s_fused": round(S / (res["fused"] * 1e-6), 1),
        "alg_bytes": alg,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_entry("decode_fused") if measured else None},
        "attention_hbm_bytes": traffic_entry("decode_attention") if measured else None,
        "core_fused_equals_pair": same,
    }
    del qry, kv, ws
    return out


def calibrate_copy(torch) -> None:
    """A plain device-to-device copy of 1 GiB (torch dispatches it to the HIP
    runtime copy kernel __amd_rocclr_copyBuffer): counter
    runs of this give the bytes-per-counter-unit factor."""
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": 2 * n}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument(
        "--workload",
        default="large_decode",
        choices=["large_decode", "large_decode_request_major"],
        help="large_decode: dense [16, 4096, 12, 512] partials; large_decode_request_major: the same "
        "sizes in the request-major layout [1024 requests, 16 splits, 4 tokens, 12, 512]",
    )
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="oracle sample size (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument(
        "--cpu-workers", type=int, default=0, help="processes for the all-cores oracle timing (default min(16, CPUs); 1 skips it)"
    )
    ap.add_argument("--all", action="store_true", help="also time the four other standard workloads (stderr)")
    ap.add_argument("--decode-kv-len", type=int, default=4096,
                    help="also time the fused split-KV decode with this many cache rows per request (0: skip)")
    ap.add_argument("--oproj-d", type=int, default=7168,
                    help="also time o_proj on the call's core with this output width (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--sizes", help="comma-separated batch sizes S: print a size sweep (one JSON object) instead")
    ap.add_argument("--splits", type=int, default=16, help="partials per (token, head) of the size sweep")
    ap.add_argument("--no-lse", action="store_true", help="size sweep of one partial without LSEs")
    ap.add_argument(
        "--traffic-from",
        nargs=4,
        metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
        help="turn rocprofv3 --pmc counter CSVs into the committed traffic figure (no GPU needed)",
    )
    ap.add_argument("--traffic-entry", choices=sorted(TRAFFIC_KERNELS),
                    help="with --traffic-from: the kernel and workload measured (default: --workload)")
    args = ap.parse_args()
    if args.traffic_from:
        entry = args.traffic_entry or args.workload
        print(json.dumps(traffic_from(*args.traffic_from, workload=entry), indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(
            "bench.py measures one GPU only: the mla_post path has no multi-GPU stage "
            "(the decode-context-parallel exchange is not implemented); run with --gpus 1.",
            file=sys.stderr,
        )
        return 2

    import torch

    import mla_split_kv_amd as m
    import synth

    # counting devices does not initialise the GPU; the oracle timings below
    # fork worker processes, which must happen before anything touches it
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        torch.cuda.set_device(0)
        m.load()
        calibrate_copy(torch)
        return 0
    if args.sizes:
        torch.cuda.set_device(0)
        m.load()
        sizes = [int(x) for x in args.sizes.split(",")]
        print(json.dumps(size_sweep(sizes, args.steps, args.warmup, m, torch, args.splits, args.no_lse)))
        return 0

    log(f"generating the {args.workload} workload (seeded, 805 MB of partials)")
    w = synth.large_decode() if args.workload == "large_decode" else synth.EXTRA[args.workload]()
    alg = algorithmic_bytes(w)

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens, one thread")
        cpu = cpu_baseline(w, args.cpu_tokens)
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        if workers > 1:
            log(f"timing the CPU oracle on {args.cpu_tokens} tokens, {workers} processes")
            cpu_all = cpu_baseline_all_cores(w, args.cpu_tokens, workers)

    torch.cuda.set_device(0)
    m.load()
    d = device_setup(w, m, torch)
    call = m.prepare(d["o"], d["lse"], d["w_v"], d["w_s"], d["gate"], d["core"], **layout_args(w))
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    t = time_gpu(call, args.steps, args.warmup, torch)
    ms_per_step = 1e3 * t["wall_s"] / args.steps
    kernel_us = 1e3 * t["event_ms"] / args.steps
    achieved = alg["alg_bytes"] / (kernel_us * 1e-6) / 1e9
    tokens_per_s = w.S * args.steps / t["wall_s"]

    copy_gbps = copy_ceiling(torch)
    rc = read_ceiling(d["o_buf"], args.steps, torch, m)
    log(f"plain read of the partial buffer: {rc}")
    op = None
    if args.oproj_d > 0:
        log(f"timing o_proj on the call's core, D = {args.oproj_d}")
        op = oproj_bench(d["core"], args.oproj_d, args.steps, args.warmup, m, torch)
        log(f"o_proj: {op}")
    extra = {}
    if args.all:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB, for cold calls
        for name in ("tiny", "no_merge", "split_merge", "dcp8"):
            wk = synth.STANDARD[name]()
            dk = device_setup(wk, m, torch)
            ck = m.prepare(dk["o"], dk["lse"], dk["w_v"], dk["w_s"], dk["gate"], dk["core"])
            tk = time_gpu(ck, 2000, 100, torch)
            ak = algorithmic_bytes(wk)
            us = 1e3 * tk["event_ms"] / 2000
            gbps = ak["alg_bytes"] / (us * 1e-6) / 1e9
            extra[name] = {
                "us_per_call": round(us, 3),
                "GBps": round(gbps, 1),
                "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "tokens_per_s": round(wk.S / (us * 1e-6), 1),
                "us_single_warm": round(time_per_call(ck, 200, torch), 3),
                "us_per_call_graph": round(time_graph(ck, torch), 3),
                "us_single_cold": round(time_per_call(ck, 100, torch, scratch), 3),
                "alg_bytes": ak["alg_bytes"],
            }
            log(f"{name}: {extra[name]}")
            del dk, ck
        del scratch
        if args.workload == "large_decode":
            wk = synth.EXTRA["large_decode_request_major"]()
            dk = device_setup(wk, m, torch)
            ck = m.prepare(dk["o"], dk["lse"], dk["w_v"], dk["w_s"], dk["gate"], dk["core"], **layout_args(wk))
            tk = time_gpu(ck, args.steps, args.warmup, torch)
            ak = algorithmic_bytes(wk)
            us = 1e3 * tk["event_ms"] / args.steps
            gbps = ak["alg_bytes"] / (us * 1e-6) / 1e9
            extra["large_decode_request_major"] = {
                "us_per_call": round(us, 3),
                "GBps": round(gbps, 1),
                "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "tokens_per_s": round(wk.S / (us * 1e-6), 1),
                "alg_bytes": ak["alg_bytes"],
            }
            log(f"large_decode_request_major: {extra['large_decode_request_major']}")
            del dk, ck

    out = {
        "metric": "tokens/s and us per mla_post call; achieved HBM GB/s vs peak (1 GPU)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_call": round(kernel_us, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "tokens": w.S,
            "splits": w.n,
            "heads": 12,
            "latent": 512,
            "v_dim": 128,
            "live_rows": alg["live_rows"],
            "rows": alg["rows"],
            "alg_bytes_per_call": alg["alg_bytes"],
            "nominal_bytes_per_call": alg["nominal_bytes"],
            "layout": "dense [16, 4096, 12, 512]" if args.workload == "large_decode"
            else "request-major [1024, 16, 4, 12, 512]",
            "parallelism": "single GPU",
            "compute": "fp32 merge of bf16 rows, MXFP4 x MXFP4 MFMA, bf16 out",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic_entry(args.workload),
        },
        "cpu_baseline": cpu,
        "copy_ceiling": {
            "GBps": round(copy_gbps, 1),
            "frac": round(achieved / copy_gbps, 4),
            "what": "plain 1 GiB device copy, bytes read + written per second",
        },
        "read_ceiling": {
            "GBps": rc["GBps"],
            "us": rc["us"],
            "frac": round(rc["us"] / kernel_us, 4),
            "what": "one streaming read of the same 805 MB partial buffer (mla_measure_read: 16-byte "
            "non-temporal loads, a contiguous chunk per workgroup), timed like the kernel; frac is its "
            "time over the kernel's",
        },
    }
    if op:
        out["oproj"] = op
    dec = None
    if args.decode_kv_len > 0:
        del d, call
        log(f"timing the fused decode (1024 x 4 tokens, 16 splits, {args.decode_kv_len} rows per request)")
        dec = decode_bench(1024, 4, 16, args.decode_kv_len, max(5, args.steps // 10), min(3, args.warmup), m, torch)
        log(f"fused decode: {dec}")
        out["fused_decode"] = dec
    if cpu_all:
        out["cpu_baseline_all_cores"] = cpu_all
    if extra:
        out["other_workloads"] = extra
    log(f"host: {platform.node()} python {platform.python_version()} torch {torch.__version__}")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
