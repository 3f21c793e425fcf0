"""bench.py's host logic on the CPU: the one-GPU guard, the algorithmic byte
count, the HBM traffic figure computed from rocprofv3 counter CSVs (scaled by
the plain copy's counters, tied to its workload and to the kernel source),
and the oracle timings' reporting fields."""

from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def run_bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=e, timeout=120)


def test_more_than_one_gpu_exits_with_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
    r = run_bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_algorithmic_bytes_large_decode():
    w = synth.large_decode()
    alg = bench.algorithmic_bytes(w)
    live = bench.live_rows(w)
    assert alg["rows"] == 16 * 4096 * 12
    assert alg["live_rows"] == live < alg["rows"]
    w_v = 12 * 128 * 256 + 12 * 128 * 16
    expect = live * 1024 + 16 * 4096 * 12 * 4 + w_v + 2 * 4096 * 1536 * 2
    assert alg["alg_bytes"] == expect == 793_979_904
    assert alg["nominal_bytes"] == 16 * 4096 * 12 * 1024 + 16 * 4096 * 12 * 4 + w_v + 2 * 4096 * 1536 * 2


def test_algorithmic_bytes_no_lse():
    w = synth.single_partial("np", 64, seed=1)
    alg = bench.algorithmic_bytes(w)
    assert alg["alg_bytes"] == 64 * 12 * 1024 + 12 * 128 * 272 + 2 * 64 * 1536 * 2


def write_counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": "C", "Counter_Value": value})


def test_traffic_from_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    k = "void (anonymous namespace)::mla_post_kernel<false, 1, 0>(KArgs, int)"
    other = "at::native::fill"
    # the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    write_counter_csv(tmp_path / "f.csv", [(k, 100.0), (k, 104.0), (k, 102.0), (other, 9e9)])
    write_counter_csv(tmp_path / "w.csv", [(k, 12.0), (k, 12.0), (other, 1.0)])
    write_counter_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", 524288.0)] * 3)
    write_counter_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", 1048576.0)] * 3)
    out = bench.traffic_from(*(str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")))
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["hbm_fetch_bytes"] == 102 * 1024 * 2  # median of the kernel's dispatches only
    assert out["hbm_write_bytes"] == 12 * 1024
    assert out["hbm_bytes_per_launch"] == 102 * 2048 + 12 * 1024
    saved = json.load(open(tmp_path / "traffic.json"))["large_decode"]
    assert saved["workload"] == "large_decode" and saved["kernel_source_sha256"] == bench.kernel_sha()
    assert bench.traffic_entry("large_decode") == out["hbm_bytes_per_launch"]
    assert bench.traffic_entry("large_decode_request_major") is None  # taken on another workload
    # a second workload's entry is added beside the first
    rm = bench.traffic_from(*(str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")),
                            workload="large_decode_request_major")
    assert bench.traffic_entry("large_decode_request_major") == rm["hbm_bytes_per_launch"]
    assert bench.traffic_entry("large_decode") == out["hbm_bytes_per_launch"]


def test_traffic_is_null_once_the_kernel_changes(tmp_path, monkeypatch):
    t = tmp_path / "traffic.json"
    t.write_text(json.dumps({"large_decode": {"workload": "large_decode", "kernel_source_sha256": "0" * 64,
                                              "hbm_bytes_per_launch": 1}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    assert bench.traffic_entry("large_decode") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_entry("large_decode") is None


def test_cpu_baselines_report_fields():
    w = synth.split_merge()
    one = bench.cpu_baseline(w, 8)
    assert one["kind"] == "oracle" and one["cores"] == 1 and one["unit"] == "tokens/s" and one["value"] > 0
    assert "first 8 of 128 tokens" in one["sample"]
    many = bench.cpu_baseline_all_cores(w, 16, 2)
    assert many["kind"] == "oracle" and many["cores"] == 2 and many["value"] > 0


def test_traffic_entries_follow_their_own_source(tmp_path, monkeypatch):
    """Each counter entry is valid only for the source file of its own kernel:
    an edit of decode.hip voids the decode entries, not mla_post's or o_proj's."""
    import shutil

    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc)
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "KERNEL_SRC", str(csrc / "mla_post.hip"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    rows = "Kernel_Name,Counter_Value\n"
    f = tmp_path / "f.csv"
    f.write_text(rows + '"x::mla_decode_kernel<false>(a)",100\n"x::oproj_big_kernel(a)",10\n"copyBuffer",524288\n')
    w = tmp_path / "w.csv"
    w.write_text(rows + '"x::mla_decode_kernel<false>(a)",50\n"x::oproj_big_kernel(a)",5\n"copyBuffer",1048576\n')
    d = bench.traffic_from(str(f), str(w), str(f), str(w), workload="decode_attention")
    o = bench.traffic_from(str(f), str(w), str(f), str(w), workload="oproj")
    assert d["hbm_bytes_per_launch"] == 100 * 2048 + 50 * 1024
    assert o["hbm_bytes_per_launch"] == 10 * 2048 + 5 * 1024
    assert bench.traffic_entry("decode_attention") == d["hbm_bytes_per_launch"]
    (csrc / "decode.hip").write_text((csrc / "decode.hip").read_text() + "\n// edited\n")
    assert bench.traffic_entry("decode_attention") is None
    assert bench.traffic_entry("oproj") == o["hbm_bytes_per_launch"]
