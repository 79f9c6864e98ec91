"""Host-side checks of the benchmark's bookkeeping (no GPU): the FLOP and byte
counts it divides by, the gate that withholds counter-measured HBM traffic once
a kernel's source has changed, and the one-GPU guard."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_exact_amd.workloads import WORKLOADS, decode_bytes, decode_flops, prefill_flops  # noqa: E402


def test_prefill_flops_follow_the_pair_counts():
    # 4*d*Hq*B FLOPs per scored (query, key) pair (QK^T and PV; the per-head
    # cost model of lesson 8 "Context Parallelism (CP)", fig. 8-1), causal
    # pairs counted exactly
    w2, w3, w4 = WORKLOADS[2], WORKLOADS[3], WORKLOADS[4]
    n = w2.S // w2.P
    for r in range(w2.P):
        # naive causal split: rank r scores r full blocks and one diagonal block
        assert prefill_flops(w2, r) == 4 * w2.d * w2.Hq * (r * n * n + n * (n + 1) // 2)
    for w in (w3, w4):
        c = w.S // (2 * w.P)
        # zig-zag: every rank the same 2Pc^2 + c pairs (lesson 8, section 4B)
        assert {prefill_flops(w, r) for r in range(w.P)} == {4 * w.d * w.Hq * (2 * w.P * c * c + c)}
        # all ranks together: the causal triangle S(S+1)/2
        assert prefill_flops(w) == 4 * w.d * w.Hq * (w.S * (w.S + 1) // 2)
    # the figure the headline rate divides by (128k-token GQA, rank 0)
    assert prefill_flops(w4, 0) == 17_592_320_262_144


def test_decode_bytes_and_flops():
    w = WORKLOADS[5]
    b = decode_bytes(w, n_parts=64)
    # K and V, each [8, 1,048,576, 8, 128] bf16, read once
    assert b["kv"] == 2 * 8 * 1_048_576 * 8 * 128 * 2 == 34_359_738_368
    rows = 8 * 64
    assert b["q"] == rows * 128 * 2
    assert b["partials"] == 64 * rows * 129 * 4
    assert b["total"] == b["kv"] + b["q"] + 2 * b["partials"] + b["out"]
    assert decode_flops(w) == 4 * 128 * rows * 1_048_576


def test_traffic_is_withheld_when_the_source_changed(tmp_path, monkeypatch):
    files = bench.PREFILL_SOURCES
    good = {"prefill": {"bytes_per_launch": 123.0, "source_hash": bench.source_hash(files)}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("prefill", files) == 123.0
    stale = {"prefill": {"bytes_per_launch": 123.0, "source_hash": "0" * 16}}
    path.write_text(json.dumps(stale))
    assert bench.measured_traffic("prefill", files) is None
    assert bench.measured_traffic("decode", bench.DECODE_SOURCES) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("prefill", files) is None


def test_source_hash_tracks_every_listed_file():
    a = bench.source_hash(["fwd_bf16.hip"])
    assert a == bench.source_hash(["fwd_bf16.hip"]) and len(a) == 16
    assert a != bench.source_hash(["fwd_bf16.hip", "ra_device.h"])


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
