#!/usr/bin/env python3
"""Benchmark of the ring-attention hot path on one MI355X.

One step runs every stage of the path once, on synthetic inputs already
resident in HBM:
  1. layout: natural -> zig-zag sharded order of Q, K, V (ra_layout_gather)
     for the 128k-token GQA workload (B1 Hq32 Hkv8 d128 S131072, P8);
  2. prefill: rank 0's share of ring attention on that workload (ra_fwd_rank_ws:
     16384 local queries x 32 heads against all 131072 keys, visited in ring
     order, causal, zig-zag);
  3. decode: KV-sharded decode (B8, 1 query, Hq64 Hkv8 d128, 1,048,576 keys
     per sequence; 8 shards, each split into 8 parts) -> per-part partials
     (ra_attn_partial), then ra_merge_partials.
Each stage is timed with HIP events on the stream the kernels run on.

The printed JSON line reports ring-attention forward TFLOP/s (exact causal
FLOPs, 4*d per scored (query, key) pair and head) as ``value``, with its
roofline against the dense bf16 MFMA peak, and the decode path's HBM GB/s in
the ``decode`` object.  ``cpu_baseline`` times the fp64 CPU oracle on a sample
of the same prefill workload.

--layout runs the same prefill shape under another split (contiguous,
striped, zigzag<k>); --prefill-cfg picks the 32k or 8k-token workload
instead; --ulysses times the whole problem as the Ulysses all-to-all scheme
beside the ring; --ring-steps times the rank share as P separate ring steps with
the state in HBM (blocks resident, and double-buffered copies on a second
stream standing in for the peer-to-peer receive); --all-ranks adds the time of every rank's share, whose maximum is
the length of one ring pass when the ranks run side by side, and of all
ranks in one launch (ra_fwd_all).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring-attn fwd TFLOP/s (% bf16 MFMA peak); KV-shard decode GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PREFILL_SOURCES = ["fwd_bf16.hip", "ra_device.h", "ra_internal.h"]
DECODE_SOURCES = ["decode.hip", "ra_device.h", "ra_internal.h"]
LAYOUT_SOURCES = ["layout.hip", "ra_device.h", "ra_internal.h"]


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "long_context_exact_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, files, key: str = "bytes_per_launch"):
    """HBM bytes per launch (or per step) from the committed rocprofv3
    counter summary, or None when the kernel source changed since the
    counters were taken."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(kernel)
    if not rec or rec.get("source_hash") != source_hash(files):
        return None
    return rec.get(key)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _affinity_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _prefill_inputs_host(w):
    from long_context_exact_amd import synthetic

    dt = w.dtype
    return (synthetic.normal_tensor(w.q_shape, w.seed(0), dt),
            synthetic.normal_tensor(w.kv_shape, w.seed(1), dt),
            synthetic.normal_tensor(w.kv_shape, w.seed(2), dt))


def cpu_prefill(w, rank=None, n_rows=None):
    """The fp64 oracle on a prefill workload: every row (rank None) or n_rows
    query rows of ``rank`` evenly spaced over its local rows (under the
    zig-zag split half from each of its two chunks); every query head, each
    row scored against all the keys it may see.  Returns (seconds, FLOPs in
    the GPU figure's convention, description)."""
    import numpy as np

    import oracle

    Q, K, V = _prefill_inputs_host(w)
    if rank is None:
        rows = np.arange(w.S, dtype=np.int64)
        what = f"all {w.S} rows"
    else:
        n = w.S // w.P
        mine = oracle.natural_positions(w.S, w.P, w.layout)[rank * n:(rank + 1) * n]
        rows = mine[np.linspace(0, n - 1, n_rows).astype(np.int64)]
        what = f"{len(rows)} query rows of rank {rank} evenly spaced over its {w.layout} rows"
    keys = rows + 1 if w.causal else np.full(rows.shape, w.S, dtype=np.int64)
    flops = 4 * w.d * w.Hq * w.B * int(np.sum(keys))
    t0 = time.perf_counter()
    oracle.attention_rows(Q, K, V, w.causal, np.zeros_like(rows), rows)
    dt = time.perf_counter() - t0
    return dt, flops, f"{what}, all {w.Hq} heads"


def cpu_decode_sequence(w, b: int = 0):
    """The fp64 oracle on one whole sequence of the decode workload: its
    query row of every head against all of its keys.  Returns (seconds,
    algorithmic K/V bytes of that sequence, FLOPs)."""
    import numpy as np

    import oracle
    from long_context_exact_amd import synthetic

    per_seq = w.S * w.Hkv * w.d
    Q = synthetic.normal_tensor(w.q_shape, w.seed(0), "bf16")[b:b + 1]
    K = synthetic.normal_range(w.seed(1), b * per_seq, (b + 1) * per_seq, "bf16").reshape(1, w.S, w.Hkv, w.d)
    V = synthetic.normal_range(w.seed(2), b * per_seq, (b + 1) * per_seq, "bf16").reshape(1, w.S, w.Hkv, w.d)
    t0 = time.perf_counter()
    oracle.attention_rows(Q, K, V, False, np.zeros(w.Sq, np.int64), np.arange(w.Sq, dtype=np.int64))
    dt = time.perf_counter() - t0
    return dt, 2 * per_seq * 2, 4 * w.d * w.Sq * w.Hq * w.S


def cpu_baseline(wp, rank: int, n_rows: int, with_legs: bool = True):
    """The oracle timed on this host's cores (every core of the affinity
    mask), on bounded samples of the workloads.  ``value`` is the headline
    prefill sample (n_rows rows of one rank's share of wp); ``legs`` adds the
    small fp32 workload and the 8k-token workload whole, a 32k-token sample,
    and one whole sequence of the decode workload."""
    import oracle
    from long_context_exact_amd.workloads import WORKLOADS

    cores = _affinity_cores()
    oracle.set_num_threads(cores)
    dt, flops, what = cpu_prefill(wp, rank, n_rows)
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "affinity_cores": cores, "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": f"{what} of {wp.name}, {flops / 1e9:.1f} GFLOP, {dt:.1f} s wall"}
    if not with_legs:
        return out
    legs = {}
    for cfg, rank_, rows_ in ((1, None, None), (2, None, None), (3, 0, 512)):
        w = WORKLOADS[cfg]
        log(f"cpu baseline: oracle on {w.name}")
        dt, flops, what = cpu_prefill(w, rank_, rows_)
        legs[w.name] = {"s": dt, "gflop": flops / 1e9, "tflops": flops / dt / 1e12,
                        "sample": what if rank_ is not None else "whole problem"}
    wd = WORKLOADS[5]
    log(f"cpu baseline: oracle on one sequence of {wd.name}")
    dt, nbytes, flops = cpu_decode_sequence(wd, 0)
    legs[wd.name] = {"s": dt, "gbs": nbytes / dt / 1e9, "tflops": flops / dt / 1e12,
                     "sample": f"sequence 0 of {wd.B}: {wd.Hq} heads x {wd.S} keys, "
                               f"{nbytes / 1e9:.2f} GB of K/V, {flops / 1e9:.1f} GFLOP"}
    out["legs"] = legs
    return out


def time_prefill_ranks(ra, torch, w, steps: int, warmup: int, dev):
    """Every rank's share of a prefill workload (ra_fwd_rank_ws with the
    automatic key-range splits) and all ranks in one launch (ra_fwd_all_ws),
    timed with HIP events on the current stream.  The maximum over ranks is
    how long one ring pass takes when the ranks run side by side."""
    from long_context_exact_amd import synthetic
    from long_context_exact_amd.workloads import prefill_flops

    dt = ra.DTYPE_BF16 if w.dtype == "bf16" else ra.DTYPE_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    nat = [synthetic.to_device(sh, w.seed(i), w.dtype, dev)
           for i, sh in ((0, w.q_shape), (1, w.kv_shape), (2, w.kv_shape))]
    Qs, Ks, Vs = (torch.empty_like(x) for x in nat)
    for a, b in zip(nat, (Qs, Ks, Vs)):
        ra.ra_layout_gather(a, b, w.S, w.P, w.layout, inverse=False)
    del nat
    n = w.S // w.P
    O_r = torch.empty(w.B, n, w.Hq, w.d, dtype=torch.float32, device=dev)
    L_r = torch.empty(w.B, w.Hq, n, dtype=torch.float32, device=dev)
    ws_r_bytes = ra.ra_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.d, w.P, False, w.causal,
                                           w.layout, dt, 0)
    ws_r = torch.empty(max(ws_r_bytes, 1), dtype=torch.uint8, device=dev)

    def timed(fn, k):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    def rank_fn(r):
        Qr = Qs[:, r * n:(r + 1) * n]
        return lambda: ra.ra_fwd_rank_ws(Qr, Ks, Vs, O_r, L_r, w.P, r, w.causal, w.layout, 0, ws_r)

    # every rank in turn for 0.3 s first: the GPU sat idle while the inputs
    # were generated on the host, and its first launches after that run slower
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.3:
        for r in range(w.P):
            rank_fn(r)()
        torch.cuda.synchronize()
    per = [timed(rank_fn(r), steps) for r in range(w.P)]
    O_all = torch.empty(w.B, w.S, w.Hq, w.d, dtype=torch.float32, device=dev)
    L_all = torch.empty(w.B, w.Hq, w.S, dtype=torch.float32, device=dev)
    ws_a_bytes = ra.ra_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.d, w.P, True, w.causal,
                                           w.layout, dt, 0)
    ws_a = torch.empty(max(ws_a_bytes, 1), dtype=torch.uint8, device=dev)
    all_ms = timed(lambda: ra.ra_fwd_all_ws(Qs, Ks, Vs, O_all, L_all, w.P, w.causal, w.layout, 0, ws_a),
                   steps)
    total = prefill_flops(w)
    rank_flops = [prefill_flops(w, r) for r in range(w.P)]
    return {"workload": w.name, "layout": w.layout,
            "rank_ms": [round(x, 4) for x in per],
            "rank_gflop": [round(f / 1e9, 2) for f in rank_flops],
            "rank_tflops": [round(f / (t * 1e-3) / 1e12, 1) for f, t in zip(rank_flops, per)],
            "slowest_rank_ms": max(per), "max_over_min": max(per) / min(per),
            "sum_of_ranks_ms": sum(per),
            "tflops_per_gpu_at_slowest_rank": total / w.P / (max(per) * 1e-3) / 1e12,
            "all_ranks_one_launch_ms": all_ms,
            "all_ranks_tflops": total / (all_ms * 1e-3) / 1e12,
            "all_ranks_frac_bf16_peak": total / (all_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "gflop_total": total / 1e9,
            "kv_splits_rank": (ws_r_bytes // (w.B * n * w.Hq * (w.d + 1) * 4)) if ws_r_bytes else 1,
            "kv_splits_all": (ws_a_bytes // (w.B * w.S * w.Hq * (w.d + 1) * 4)) if ws_a_bytes else 1}


def sample_sclk(fn, seconds: float = 3.0):
    """Run fn back to back for about `seconds` while a child rocm-smi samples
    the shader clock.  Returns the MHz readings (empty without rocm-smi, and
    under rocprofv3, whose tool library would initialise the GPU in the child
    before rocm-smi's interpreter starts)."""
    import re
    import shutil
    import subprocess
    import threading

    import torch

    smi = shutil.which("rocm-smi")
    if smi is None or any(k.startswith("ROCPROF") for k in os.environ):
        return []
    readings = []

    def sampler():
        for _ in range(4):
            time.sleep(seconds / 5)
            try:
                r = subprocess.run([smi, "--showclocks"], capture_output=True, text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                continue
            for line in r.stdout.splitlines():
                if "sclk" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, flags=re.I)
                    if m:
                        readings.append(int(m.group(1)))
                        break

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < 3 * seconds:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    th.join()
    return readings


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rank", type=int, default=0, help="prefill rank whose share is timed")
    ap.add_argument("--decode-parts", type=int, default=64)
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="query rows of the timed rank in the CPU oracle's headline sample")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip timing every rank and the all-ranks launch of the 8k and 32k-token "
                         "prefill workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-cfg", type=int, choices=[2, 3, 4], default=4,
                    help="prefill workload: 4 = 128k-token GQA (default, the headline), 3 = 32k "
                         "zig-zag MHA, 2 = 8k contiguous MHA")
    ap.add_argument("--all-ranks", action="store_true",
                    help="also time every rank's share of the prefill (the ring step lasts as "
                         "long as the slowest rank)")
    ap.add_argument("--decode-rr-block", type=int, default=0,
                    help="decode over the KV cache dealt round-robin in blocks of this many tokens "
                         "to the 8 shard caches (built by ra_kv_append_rr before timing); 0 = one "
                         "contiguous cache per sequence (default)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock while the prefill runs back to back")
    ap.add_argument("--ulysses", action="store_true",
                    help="also time the whole prefill problem as DeepSpeed Ulysses on one GPU: "
                         "all-to-all of Q, K, V to head groups, full-sequence attention of all "
                         "groups, all-to-all of O and LSE back; beside the ring (ra_fwd_all_ws)")
    ap.add_argument("--ring-steps", action="store_true",
                    help="also time the timed rank's share as P ring steps (ra_ring_step) on one "
                         "stream, and double-buffered with the next block copied on a second stream")
    ap.add_argument("--layout", default=None,
                    help="prefill split: the workload's own (zig-zag, default) or another one "
                         "(contiguous, striped, zigzag<k>) on the same shape")
    ap.add_argument("--workload", choices=["all", "prefill", "decode", "copy"], default="all",
                    help="copy: a plain 1 GiB device copy through the layout kernel (contiguous "
                         "layout), used to calibrate the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the ring is "
              "simulated on a single MI355X, with every shard resident; no multi-GPU run exists.",
              file=sys.stderr)
        return 2

    import torch

    import long_context_exact_amd as ra
    from long_context_exact_amd import synthetic
    from long_context_exact_amd.workloads import WORKLOADS, decode_bytes, prefill_flops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ra.lib()
    dev = torch.device("cuda:0")
    do_pre = args.workload in ("all", "prefill")
    do_dec = args.workload in ("all", "decode")
    if args.workload == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            ra.ra_layout_gather(src, dst, 1 << 20, 1, "contiguous", inverse=False, outer=1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            ra.ra_layout_gather(src, dst, 1 << 20, 1, "contiguous", inverse=False, outer=1)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"workload": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "ms": ms, "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)
        return 0
    wp, wd = WORKLOADS[args.prefill_cfg], WORKLOADS[5]
    own_layout = (args.layout is None or args.layout == wp.layout) and args.prefill_cfg == 4
    if args.layout is not None:
        wp = dataclasses.replace(wp, layout=args.layout)

    launches = []  # (stage, fn)
    if do_pre:
        log(f"generating prefill inputs {wp.name}")
        Qn = synthetic.to_device(wp.q_shape, wp.seed(0), "bf16", dev)
        Kn = synthetic.to_device(wp.kv_shape, wp.seed(1), "bf16", dev)
        Vn = synthetic.to_device(wp.kv_shape, wp.seed(2), "bf16", dev)
        Qs, Ks, Vs = torch.empty_like(Qn), torch.empty_like(Kn), torch.empty_like(Vn)
        n = wp.S // wp.P
        r = args.rank
        Q_r = Qs[:, r * n:(r + 1) * n]
        O_r = torch.empty(Q_r.shape, dtype=torch.float32, device=dev)  # fp32 accumulator output
        L_r = torch.empty(wp.B, wp.Hq, n, dtype=torch.float32, device=dev)
        # workspace for the automatic key-range splits (none for the 128k
        # workload, whose rank share already has 2048 query tiles)
        ws_r_bytes = ra.ra_fwd_workspace_bytes(wp.B, wp.Hq, wp.Hkv, wp.S, wp.d, wp.P, False,
                                               wp.causal, wp.layout, ra.DTYPE_BF16, 0)
        ws_r = torch.empty(max(ws_r_bytes, 1), dtype=torch.uint8, device=dev)
        splits_r = ws_r_bytes // (wp.B * n * wp.Hq * (wp.d + 1) * 4) if ws_r_bytes else 1

        def layout():
            for a, b in ((Qn, Qs), (Kn, Ks), (Vn, Vs)):
                ra.ra_layout_gather(a, b, wp.S, wp.P, wp.layout, inverse=False)

        def prefill():
            ra.ra_fwd_rank_ws(Q_r, Ks, Vs, O_r, L_r, wp.P, r, wp.causal, wp.layout, 0, ws_r)

        launches += [("layout", layout), ("prefill", prefill)]
    if do_dec:
        log(f"generating decode inputs {wd.name} (2 x 16 GiB)")
        Qd = synthetic.to_device(wd.q_shape, wd.seed(0), "bf16", dev)
        Kd = synthetic.to_device(wd.kv_shape, wd.seed(1), "bf16", dev)
        Vd = synthetic.to_device(wd.kv_shape, wd.seed(2), "bf16", dev)
        parts = args.decode_parts
        rows = wd.B * wd.Sq * wd.Hq
        Op = torch.empty(parts, rows, wd.d, dtype=torch.float32, device=dev)
        lp = torch.empty(parts, rows, dtype=torch.float32, device=dev)
        Od = torch.empty(rows, wd.d, dtype=torch.float32, device=dev)
        ld = torch.empty(rows, dtype=torch.float32, device=dev)

        rr = args.decode_rr_block
        if rr > 0:
            # the cache a KV-parallel group builds by appending blocks in turn
            cap = max(len(range(sh * rr, wd.S, wd.P * rr)) * rr for sh in range(wd.P)) + rr
            Kc = torch.empty(wd.P, wd.B, cap, wd.Hkv, wd.d, dtype=torch.bfloat16, device=dev)
            Vc = torch.empty_like(Kc)
            torch.cuda.synchronize()
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record()
            ra.ra_kv_append_rr(Kc, Vc, Kd, Vd, 0, rr)  # the whole 1M-token cache in one call
            eb.record()
            torch.cuda.synchronize()
            bulk_ms = ea.elapsed_time(eb)
            del Kd, Vd
            if parts % wd.P:
                raise SystemExit("--decode-parts must be a multiple of the 8 shards")

            def decode():
                ra.ra_attn_partial_rr(Qd, Kc, Vc, Op, lp, wd.S, rr, parts // wd.P)
        else:
            def decode():
                ra.ra_attn_partial(Qd, Kd, Vd, Op, lp, parts)

        def merge():
            ra.ra_merge_partials(Op, lp, Od, ld)

        launches += [("decode", decode), ("merge", merge)]
    torch.cuda.synchronize()

    def step(events=None):
        for i, (_, fn) in enumerate(launches):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = {name: sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
                for i, (name, _) in enumerate(launches)}
    ms = {name: sum(v) / len(v) for name, v in per_step.items()}
    med = {name: v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
           for name, v in per_step.items()}
    mn = {name: v[0] for name, v in per_step.items()}
    log("stage ms: " + ", ".join(f"{k}={v:.3f}" for k, v in ms.items()))

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic i.i.d. N(0,1) inputs rounded to bf16 (seeded numpy PCG64)"}
    cfg = {}
    if do_pre:
        flops = prefill_flops(wp, rank=args.rank)
        tflops = flops / (ms["prefill"] * 1e-3) / 1e12
        lay_bytes = 2 * 2 * (wp.B * wp.S * (wp.Hq + 2 * wp.Hkv) * wp.d)  # read + write, bf16
        out.update({"value": tflops, "unit": "TFLOP/s"})
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                           "traffic": (measured_traffic("prefill", PREFILL_SOURCES)
                                       if own_layout else None),
                           "kernel": "fwd_bf16_kernel<128>", "flops_per_launch": flops,
                           "ms_per_launch": ms["prefill"], "ms_median": med["prefill"],
                           "ms_min": mn["prefill"], "kv_splits": splits_r}
        out["layout"] = {"value": lay_bytes / (ms["layout"] * 1e-3) / 1e9, "unit": "GB/s",
                         "ms": ms["layout"], "bytes": lay_bytes,
                         "traffic": (measured_traffic("layout", LAYOUT_SOURCES, "bytes_per_step")
                                     if own_layout else None),
                         "frac_hbm": lay_bytes / (ms["layout"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
        cfg.update({"workload": f"{wp.name} rank-{args.rank} share", "global_batch": wp.B,
                    "seq_len": wp.S, "heads_q": wp.Hq, "heads_kv": wp.Hkv, "head_dim": wp.d,
                    "ranks": wp.P, "layout": wp.layout, "causal": wp.causal})
    if do_dec:
        nb = decode_bytes(wd, args.decode_parts)
        gbs = nb["attn_partial"] / (ms["decode"] * 1e-3) / 1e9
        tot = nb["total"] / ((ms["decode"] + ms["merge"]) * 1e-3) / 1e9
        out["decode"] = {"value": tot, "unit": "GB/s", "frac_hbm": tot / PEAK_HBM_GBS,
                         "ms": ms["decode"] + ms["merge"],
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": measured_traffic("decode", DECODE_SOURCES),
                                      "kernel": "decode_bf16_kernel<128>",
                                      "bytes_per_launch": nb["attn_partial"],
                                      "ms_per_launch": ms["decode"], "ms_median": med["decode"],
                                      "ms_min": mn["decode"]},
                         "merge_ms": ms["merge"], "parts": args.decode_parts}
        cfg["decode_workload"] = wd.name
        if rr > 0:
            # one decode step's append: one new token per sequence
            newK = torch.zeros(wd.B, 1, wd.Hkv, wd.d, dtype=torch.bfloat16, device=dev)
            for _ in range(args.warmup):
                ra.ra_kv_append_rr(Kc, Vc, newK, newK, wd.S, rr)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                ra.ra_kv_append_rr(Kc, Vc, newK, newK, wd.S, rr)
            e1.record()
            torch.cuda.synchronize()
            kv_bytes = 2 * wd.B * wd.S * wd.Hkv * wd.d * 2
            out["decode"]["cache"] = {"layout": f"round-robin blocks of {rr} tokens over {wd.P} shards",
                                      "append_one_token_ms": e0.elapsed_time(e1) / args.steps,
                                      "bulk_append_ms": bulk_ms,
                                      "bulk_append_GBps": 2 * kv_bytes / (bulk_ms * 1e-3) / 1e9}
            cfg["decode_workload"] = f"{wd.name} round-robin cache (blocks of {rr})"
        if not do_pre:
            out.update({"value": tot, "unit": "GB/s", "roofline": out["decode"]["roofline"]})
            cfg["workload"] = wd.name
    cfg["parallelism"] = "simulated ring (8 ranks resident on 1 GPU)"
    out["config"] = cfg
    if do_pre and not args.no_clock:
        log("sampling the shader clock while the prefill runs back to back")
        mhz = sample_sclk(prefill)
        if mhz:
            med = sorted(mhz)[len(mhz) // 2]
            attainable = PEAK_BF16_TFLOPS * med / 2400.0
            out["roofline"]["clock"] = {
                "sclk_mhz_samples": mhz, "sclk_mhz_median": med,
                "peak_at_this_clock_tflops": attainable,
                "frac_at_this_clock": out["roofline"]["achieved"] / attainable,
                "note": "rocm-smi in a child process while the rank share runs back to back; the "
                        "published peak is quoted at 2400 MHz"}
    if do_pre and args.all_ranks:
        log(f"timing each of the {wp.P} ranks, {args.steps} launches each")
        per = []
        for rr in range(wp.P):
            Qrr = Qs[:, rr * n:(rr + 1) * n]
            for _ in range(args.warmup):
                ra.ra_fwd_rank_ws(Qrr, Ks, Vs, O_r, L_r, wp.P, rr, wp.causal, wp.layout, 0, ws_r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                ra.ra_fwd_rank_ws(Qrr, Ks, Vs, O_r, L_r, wp.P, rr, wp.causal, wp.layout, 0, ws_r)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / args.steps)
        total = prefill_flops(wp)
        # all ranks in one launch: the whole problem on this one GPU
        O_all = torch.empty(wp.B, wp.S, wp.Hq, wp.d, dtype=torch.float32, device=dev)
        L_all = torch.empty(wp.B, wp.Hq, wp.S, dtype=torch.float32, device=dev)
        ws_a_bytes = ra.ra_fwd_workspace_bytes(wp.B, wp.Hq, wp.Hkv, wp.S, wp.d, wp.P, True,
                                               wp.causal, wp.layout, ra.DTYPE_BF16, 0)
        ws_a = torch.empty(max(ws_a_bytes, 1), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            ra.ra_fwd_all_ws(Qs, Ks, Vs, O_all, L_all, wp.P, wp.causal, wp.layout, 0, ws_a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            ra.ra_fwd_all_ws(Qs, Ks, Vs, O_all, L_all, wp.P, wp.causal, wp.layout, 0, ws_a)
        e1.record()
        torch.cuda.synchronize()
        all_ms = e0.elapsed_time(e1) / args.steps
        splits_a = ws_a_bytes // (wp.B * wp.S * wp.Hq * (wp.d + 1) * 4) if ws_a_bytes else 1
        del O_all, L_all, ws_a
        out["fwd_all"] = {"ms": all_ms, "tflops": total / (all_ms * 1e-3) / 1e12,
                          "kv_splits": splits_a}
        out["ranks"] = {"ms": [round(x, 4) for x in per], "ring_step_ms": max(per),
                        "max_over_min": max(per) / min(per),
                        "gflop": [round(prefill_flops(wp, rr) / 1e9, 1) for rr in range(wp.P)],
                        "tflops_per_gpu_at_ring_step": total / wp.P / (max(per) * 1e-3) / 1e12}
    if do_pre and args.ring_steps:
        log(f"timing rank {r} as {wp.P} ring steps")
        O_s = torch.empty(Q_r.shape, dtype=torch.float32, device=dev)
        L_s = torch.empty_like(L_r)
        Q_rc = Q_r.contiguous()

        def block(x, s_):
            return x[:, s_ * n:(s_ + 1) * n]

        def step_plain(Kb, Vb, t):
            ra.ra_ring_step(Q_rc, Kb, Vb, O_s, L_s, wp.S, wp.P, r, t, wp.causal, wp.layout)

        def step_split(Kb, Vb, t):  # automatic key-range splits through the rank's workspace
            ra.ra_ring_step_ws(Q_rc, Kb, Vb, O_s, L_s, wp.S, wp.P, r, t, wp.causal, wp.layout, 0, ws_r)

        def steps_resident(step=step_plain):
            for t in range(wp.P):
                s_ = (r - t) % wp.P
                step(block(Ks, s_), block(Vs, s_), t)

        comp = torch.cuda.current_stream()
        copy = torch.cuda.Stream()
        bufK = [torch.empty(block(Ks, 0).shape, dtype=Ks.dtype, device=dev) for _ in range(2)]
        bufV = [torch.empty_like(bufK[0]) for _ in range(2)]
        arrived = [torch.cuda.Event() for _ in range(2)]
        free = [torch.cuda.Event() for _ in range(2)]

        def receive(t):
            s_ = (r - t) % wp.P
            with torch.cuda.stream(copy):
                copy.wait_event(free[t % 2])
                bufK[t % 2].copy_(block(Ks, s_))
                bufV[t % 2].copy_(block(Vs, s_))
                arrived[t % 2].record(copy)

        def steps_double_buffered(step=step_plain):
            for e in free:
                e.record(comp)
            receive(0)
            for t in range(wp.P):
                if t + 1 < wp.P:
                    receive(t + 1)
                comp.wait_event(arrived[t % 2])
                step(bufK[t % 2], bufV[t % 2], t)
                free[t % 2].record(comp)

        def time_fn(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        t_graph = t_res_split = None
        if wp.B == 1:  # a shard of a [1, S, H, d] tensor is a contiguous block
            t_res = time_fn(steps_resident)
            t_res_split = time_fn(lambda: steps_resident(step_split))
            # the same P launches captured once and replayed (no allocation, no memset inside)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                steps_resident()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                steps_resident()
            torch.cuda.synchronize()
            t_graph = time_fn(graph.replay)
        else:
            t_res = None
        t_db = time_fn(steps_double_buffered)
        t_db_split = time_fn(lambda: steps_double_buffered(step_split))
        # the rank share in one launch, timed again here with the GPU as warm as for the steps
        # (a short workload's headline figure can be taken before the clock has ramped up)
        t_fused = time_fn(prefill)
        blk_bytes = 2 * bufK[0].numel() * bufK[0].element_size()
        out["ring_steps"] = {"steps": wp.P, "resident_ms": t_res, "graph_replay_ms": t_graph,
                             "double_buffered_ms": t_db,
                             "fused_ms": t_fused, "block_bytes_per_step": blk_bytes,
                             "overhead_vs_fused": t_db / t_fused - 1.0,
                             "overhead_resident_vs_fused": t_res / t_fused - 1.0 if t_res else None,
                             # the library's automatic count for a step: the rank share's,
                             # capped at one range per 1024 keys of the block
                             "kv_splits": max(1, min(splits_r, n // 1024)), "resident_split_ms": t_res_split,
                             "double_buffered_split_ms": t_db_split,
                             "overhead_vs_fused_split": t_db_split / t_fused - 1.0,
                             "overhead_resident_vs_fused_split": t_res_split / t_fused - 1.0 if t_res_split else None}
        del O_s, L_s, bufK, bufV
    if do_pre and args.ulysses:
        P_, B_, S_ = wp.P, wp.B, wp.S
        if wp.Hq % P_ or wp.Hkv % P_:
            raise SystemExit("Ulysses needs the heads to divide by the ranks")
        log("timing the Ulysses all-to-all scheme and the ring on the whole problem")
        Qh = torch.empty(P_ * B_, S_, wp.Hq // P_, wp.d, dtype=torch.bfloat16, device=dev)
        Kh = torch.empty(P_ * B_, S_, wp.Hkv // P_, wp.d, dtype=torch.bfloat16, device=dev)
        Vh = torch.empty_like(Kh)
        Oh = torch.empty(P_ * B_, S_, wp.Hq // P_, wp.d, dtype=torch.float32, device=dev)
        Lh = torch.empty(P_ * B_, wp.Hq // P_, S_, dtype=torch.float32, device=dev)
        O_n = torch.empty(B_, S_, wp.Hq, wp.d, dtype=torch.float32, device=dev)
        L_n = torch.empty(B_, wp.Hq, S_, dtype=torch.float32, device=dev)
        wsu_bytes = ra.ra_fwd_workspace_bytes(P_ * B_, wp.Hq // P_, wp.Hkv // P_, S_, wp.d, 1, True,
                                              wp.causal, "contiguous", ra.DTYPE_BF16, 0)
        wsu = torch.empty(max(wsu_bytes, 1), dtype=torch.uint8, device=dev)
        qrun, kvrun = wp.Hq // P_ * wp.d * 2, wp.Hkv // P_ * wp.d * 2

        def u_in():
            ra.ra_head_a2a(Qn, Qh, B_, S_, P_, qrun, False)
            ra.ra_head_a2a(Kn, Kh, B_, S_, P_, kvrun, False)
            ra.ra_head_a2a(Vn, Vh, B_, S_, P_, kvrun, False)

        def u_attn():
            ra.ra_fwd_all_ws(Qh, Kh, Vh, Oh, Lh, 1, wp.causal, "contiguous", 0, wsu)

        def u_out():
            ra.ra_head_a2a(Oh, O_n, B_, S_, P_, wp.Hq // P_ * wp.d * 4, True)
            ra.ra_head_a2a(Lh, L_n, B_, 1, P_, wp.Hq // P_ * S_ * 4, True)

        O_all = torch.empty(B_, S_, wp.Hq, wp.d, dtype=torch.float32, device=dev)
        L_all = torch.empty(B_, wp.Hq, S_, dtype=torch.float32, device=dev)
        wsr_bytes = ra.ra_fwd_workspace_bytes(B_, wp.Hq, wp.Hkv, S_, wp.d, P_, True, wp.causal,
                                              wp.layout, ra.DTYPE_BF16, 0)
        wsr = torch.empty(max(wsr_bytes, 1), dtype=torch.uint8, device=dev)

        def ring_all():
            ra.ra_fwd_all_ws(Qs, Ks, Vs, O_all, L_all, P_, wp.causal, wp.layout, 0, wsr)

        def tfn(fn, k):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(k):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / k

        k_ = max(1, min(args.steps, 3))
        t_in, t_attn, t_out = tfn(u_in, k_), tfn(u_attn, k_), tfn(u_out, k_)
        t_ring = tfn(ring_all, k_)
        total = prefill_flops(wp)
        n_ = S_ // P_
        eb = 2
        # per rank during attention: ring = Q_r, own K/V shard, one received K/V
        # block, fp32 O_r; Ulysses = the rank's sequence shard of Q/K/V (the
        # all-to-all's send side), its head group of Q/K/V for the whole
        # sequence, fp32 O of that head group
        ring_mem = (n_ * wp.Hq * wp.d * eb + 2 * (2 * n_ * wp.Hkv * wp.d * eb)
                    + n_ * wp.Hq * wp.d * 4) * B_
        uly_mem = (n_ * (wp.Hq + 2 * wp.Hkv) * wp.d * eb + S_ * (wp.Hq + 2 * wp.Hkv) // P_ * wp.d * eb
                   + S_ * wp.Hq // P_ * wp.d * 4) * B_
        out["ulysses"] = {
            "a2a_in_ms": t_in, "attention_ms": t_attn, "a2a_out_ms": t_out,
            "total_ms": t_in + t_attn + t_out, "ring_fwd_all_ms": t_ring,
            "tflops_ulysses": total / ((t_in + t_attn + t_out) * 1e-3) / 1e12,
            "tflops_ring": total / (t_ring * 1e-3) / 1e12,
            "per_rank_bytes_ring": ring_mem, "per_rank_bytes_ulysses": uly_mem,
            "note": "one GPU: the all-to-all is a local transposition; the ring's block exchange is "
                    "not simulated (all shards resident)"}
        del Qh, Kh, Vh, Oh, Lh, O_n, L_n, O_all, L_all, wsu, wsr
    if do_pre and not args.no_other_prefill and args.prefill_cfg == 4 and args.layout is None:
        # the 8k-token naive split and the 32k-token zig-zag split: per-rank
        # balance and the all-ranks time (parity-tested workloads, not the headline)
        out["other_prefill"] = {}
        for c in (2, 3):
            log(f"timing every rank of {WORKLOADS[c].name}")
            out["other_prefill"][f"cfg{c}"] = time_prefill_ranks(ra, torch, WORKLOADS[c], args.steps,
                                                                 args.warmup, dev)
    if do_pre and not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} sampled rows and the other workloads' samples")
        out["cpu_baseline"] = cpu_baseline(wp, args.rank, args.cpu_rows,
                                           with_legs=args.prefill_cfg == 4 and args.layout is None)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
