"""Benchmark: packed QSA decode on one MI355X.

Workload (default): bs=128 rows, 24 Q heads over 2 KV heads, head dim 256,
bf16 pools [262144 slots, 2, 256] ~ N(0, 1) with 5% of the key rows scaled
x8, every row at 2055 selected entries drawn uniformly with replacement.
Inputs are resident in HBM before timing starts.  One step = one
qsa_decode call (one kernel launch).  Several index banks (same recipe,
different seeds) rotate between steps so that consecutive steps do not
re-read the same rows from the caches.

Prints one JSON line.  value = gathered-KV bytes / time (GB/s), where
gathered-KV bytes = sum_b L_b * Hkv * 2 (K and V) * 512 B.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode µs/call + gathered-KV GB/s (% HBM peak), bs 1–128, sel≤2055"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "sparse_index_paged_amd", "csrc", "qsa_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qsa_decode_bs128_tp1_bf16_traffic.md")


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per launch measured with rocprofv3 --pmc for the current
    kernel source, or None if absent / taken on another kernel version."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    m = re.search(r"TRAFFIC_JSON:\s*(\{.*\})", open(TRAFFIC_FILE).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def gathered_bytes(lengths, hkv: int, row_bytes: int = 512) -> int:
    return int(sum(int(x) for x in lengths)) * hkv * 2 * row_bytes


def cpu_baseline(case, min_seconds: float):
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    used = oracle.threads_used(threads)
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode(case.q, case.k_pool, case.v_pool, case.sel, case.cu, nthreads=threads)
        calls += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    b = gathered_bytes(case.lengths, case.hkv) * calls
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"the full workload (all {case.bs} rows) decoded {calls}x by the float64 "
                      f"oracle with {used} OpenMP threads, {dt:.1f} s wall; "
                      f"{dt / calls * 1e6:.0f} us per call"}


def copy_mode(args):
    """Plain device copy of known size (calibrates rocprofv3 byte counters)."""
    import torch
    n = args.copy_mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": dt * 1e3, "GBps_rw": 2 * n * 4 / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--banks", type=int, default=4)
    ap.add_argument("--bs", type=int, default=128)
    ap.add_argument("--hkv", type=int, default=2, choices=[1, 2])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["decode", "copy"], default="decode")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--split-target", type=int, default=None)
    ap.add_argument("--min-split-keys", type=int, default=None)
    ap.add_argument("--waves", type=int, default=None)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(the decode shards by row or KV head with no exchange); run with "
                         "--gpus 1\n")
        sys.exit(2)

    import torch
    if args.mode == "copy":
        copy_mode(args)
        return

    import numpy as np

    import sparse_index_paged_amd as qsa
    import synth

    if args.split_target:
        qsa.set_option("split_target", args.split_target)
    if args.min_split_keys:
        qsa.set_option("min_split_keys", args.min_split_keys)
    if args.waves:
        qsa.set_option("waves_per_workgroup", args.waves)

    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    case = synth.case_bs128_tp1_saturated(bs=args.bs, hkv=args.hkv)
    bank_sels = [case.sel]
    for i in range(1, args.banks):
        rng = np.random.default_rng(103_000 + i)
        lists = [synth.draw_indices(rng, n, case.k_pool.shape[0]) for n in case.lengths]
        bank_sels.append(synth.pack(lists)[0])
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)

    q = case.q.cuda()
    k = case.k_pool.cuda()
    v = case.v_pool.cuda()
    cu = torch.from_numpy(case.cu).cuda()
    sels = [torch.from_numpy(s).cuda() for s in bank_sels]
    out = torch.empty(case.bs, case.hq, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.bs, case.hq, dtype=torch.float32, device="cuda")
    qsa.workspace_reserve(case.bs, case.hq, case.hkv)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        qsa.decode(q, k, v, sels[i % len(sels)], cu, out=out, lse=lse)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        qsa.decode(q, k, v, sels[i % len(sels)], cu, out=out, lse=lse)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    counters_ok = all(c == 0 for c in qsa.debug_counters())

    b_kv = gathered_bytes(case.lengths, case.hkv)
    gbs = b_kv / (ms_per_step * 1e-3) / 1e9
    splits, wgs = qsa.plan(case.bs, case.hkv)
    traffic = committed_traffic()

    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(ms_per_step * 1e3, 3),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"packed QSA decode bs={case.bs} "
                        f"{'TP1 (24Q/2KV' if case.hkv == 2 else 'TP2 (12Q/1KV'}, D=256) bf16 pools "
                        f"[262144,{case.hkv},256], 2055 selected slots per row, 5% keys x8",
            "bs": case.bs, "hq": case.hq, "hkv": case.hkv, "head_dim": 256,
            "sel_per_row": int(case.lengths.max()), "pool_slots": int(case.k_pool.shape[0]),
            "index_banks": len(sels), "splits": splits, "workgroups": wgs,
            "gathered_kv_bytes_per_call": b_kv, "counters_at_rest": counters_ok,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": b_kv,
            "kernel": "qsa_decode_kernel<bf16>",
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
