"""Benchmark: packed QSA decode on one MI355X.

Workload (default): bs=128 rows, 24 Q heads over 2 KV heads, head dim 256,
bf16 pools [262144 slots, 2, 256] ~ N(0, 1) with 5% of the key rows scaled
x8, every row at 2055 selected entries drawn uniformly with replacement.
Inputs are resident in HBM before timing starts.  One step = one
qsa_decode call (one kernel launch).  Several index banks (same recipe,
different seeds) rotate between steps so that consecutive steps do not
re-read the same rows from the caches.  K timed eager launches, 5 repeats,
median (``--timing graph`` times the K steps captured once into a HIP graph
and replayed instead; on this stack that is slightly slower, not faster).

Prints one JSON line.  value = gathered-KV bytes / time (GB/s), where
gathered-KV bytes = sum_b L_b * Hkv * 2 (K and V) * 512 B.

Other lines (not the default run): ``--kv-format fp8|int8|int4`` decodes
from quantized pools (written on the device by qsa_kv_store from the same
bf16 pools; gathered bytes then count codes + scales), ``--kv-format
tiered`` decodes from a tiered pool (int4-g32 pool plus an int8-g64 ring of
``--ring-rows`` rows, written by qsa_kv_store_tiered in slot order, so the
ring holds the last ring-rows slots; ``--hot-frac`` draws that fraction of
the entries from those slots, otherwise the lists are the default uniform
ones), ``--mode store`` times qsa_kv_store itself, and ``--mode configs`` prints
one line per measured workload configuration (see configs_mode).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

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


COUNTERS_FILE = os.path.join(ROOT, "profiles", "qsa_decode_bs128_tp1_bf16_counters.md")


def committed_mfma_busy():
    """MFMA busy share (%) from the committed shader-counter summary of the
    current kernel source, or None if absent / taken on another version."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    sha = re.search(r"Kernel source sha256\[:16\] = `([0-9a-f]+)`", text)
    busy = re.search(r"MFMA busy share = .*?= ([0-9.]+) %", text, re.S)
    if not sha or not busy or sha.group(1) != kernel_sha():
        return None
    return float(busy.group(1))


def gathered_bytes(lengths, hkv: int, row_bytes: int = 512) -> int:
    return int(sum(int(x) for x in lengths)) * hkv * 2 * row_bytes


FORMATS = {  # kv format -> (pool elements per row, bytes per element, default group, torch dtype)
    "bf16": (256, 2, 256, "bfloat16"),
    "fp8": (256, 1, 256, "uint8"),
    "int8": (256, 1, 64, "int8"),
    "int4": (128, 1, 32, "uint8"),
}


def row_bytes(fmt: str, group: int, scale_bytes: int) -> int:
    """Bytes one (slot, KV head) row occupies in the pools: codes + scales."""
    code = FORMATS[fmt][0] * FORMATS[fmt][1]
    return code if fmt == "bf16" else code + (256 // group) * scale_bytes


def quantized_pools(k, v, fmt, group, scale_dtype):
    """Device pools of `fmt` written by qsa_kv_store from bf16 device pools
    (every slot, in slot order)."""
    import torch
    import sparse_index_paged_amd as qsa
    slots, hkv = k.shape[0], k.shape[1]
    pdt = getattr(torch, FORMATS[fmt][3])
    kc = torch.empty((slots, hkv, FORMATS[fmt][0]), dtype=pdt, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((slots, hkv, 256 // group), dtype=scale_dtype, device="cuda")
    vs = torch.empty_like(ks)
    loc = torch.arange(slots, dtype=torch.int32, device="cuda")
    qsa.kv_store(k, v, loc, kc, vc, kv_format=fmt, k_scale=ks, v_scale=vs, group_size=group)
    torch.cuda.synchronize()
    return kc, vc, ks, vs


def tiered_pools(k, v, ring_rows):
    """Tiered device pool written by qsa_kv_store_tiered from bf16 device
    pools, every slot in slot order (calls of 32768 tokens)."""
    import torch
    import sparse_index_paged_amd as qsa
    slots, hkv = k.shape[0], k.shape[1]
    dev = "cuda"
    pool = dict(
        ring_k=torch.empty((ring_rows, hkv, 256), dtype=torch.int8, device=dev),
        ring_v=torch.empty((ring_rows, hkv, 256), dtype=torch.int8, device=dev),
        ring_k_scale=torch.empty((ring_rows, hkv, 4), dtype=torch.float16, device=dev),
        ring_v_scale=torch.empty((ring_rows, hkv, 4), dtype=torch.float16, device=dev),
        owner=torch.full((ring_rows,), -1, dtype=torch.int32, device=dev),
        claim=torch.zeros((ring_rows,), dtype=torch.int32, device=dev),
        cold_k=torch.empty((slots, hkv, 128), dtype=torch.uint8, device=dev),
        cold_v=torch.empty((slots, hkv, 128), dtype=torch.uint8, device=dev),
        cold_k_scale=torch.empty((slots, hkv, 8), dtype=torch.float16, device=dev),
        cold_v_scale=torch.empty((slots, hkv, 8), dtype=torch.float16, device=dev))
    for b0 in range(0, slots, 32768):
        loc = torch.arange(b0, min(slots, b0 + 32768), dtype=torch.int32, device=dev)
        qsa.kv_store_tiered(k[b0:b0 + 32768], v[b0:b0 + 32768], loc, pool)
    torch.cuda.synchronize()
    return pool


def tiered_gathered_bytes(sel, cu, owner, hkv):
    """Bytes a tiered decode must read: per (entry, KV head) its owner id
    (4 B) plus K and V of the tier it reads (ring: 256 codes + 4 fp16
    scales; int4 pool: 128 bytes + 8 fp16 scales)."""
    import numpy as np
    s = sel[: int(cu[-1])].astype(np.int64)
    hot = owner[s & (len(owner) - 1)] == s
    n_hot = int(hot.sum())
    n_cold = int(s.size - n_hot)
    per_head = n_hot * (2 * (256 + 8) + 4) + n_cold * (2 * (128 + 16) + 4)
    return per_head * hkv, n_hot / max(1, s.size)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, min_seconds: float):
    """The float64 oracle on the host: the whole workload with the host's
    threads (at most 16), repeated for about min_seconds, and a bounded
    sample (8 rows) with one thread."""
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
    rows = min(8, case.bs)
    cu1 = case.cu[: rows + 1]
    t1 = time.perf_counter()
    oracle.decode(case.q[:rows].contiguous(), case.k_pool, case.v_pool, case.sel[: int(cu1[-1])], cu1,
                  nthreads=1)
    dt1 = time.perf_counter() - t1
    b1 = gathered_bytes(np.diff(cu1), case.hkv)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"the full workload (all {case.bs} rows) decoded {calls}x by the float64 "
                      f"oracle with {used} OpenMP threads, {dt:.1f} s wall; "
                      f"{dt / calls * 1e6:.0f} us per call",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": round(b1 / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"the first {rows} rows, once, 1 thread, {dt1:.2f} s"}}


def copy_rate(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Plain device-to-device copy on the same box (read + write GB/s)."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / reps / 1e3
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / sec / 1e9


_PROBE = None


def probe_lib():
    """libqsa_probe.so (the bare gather), or None if it was not built."""
    global _PROBE
    if _PROBE is None:
        import ctypes
        path = os.path.join(ROOT, "sparse_index_paged_amd", "libqsa_probe.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.qsa_probe_gather.restype = ctypes.c_int
        lib.qsa_probe_gather.argtypes = [P, P, I64, I64, ctypes.c_int, ctypes.c_int, P, I64, I64, I64,
                                         P, I64, P]
        lib.qsa_probe_line_reads.restype = ctypes.c_int
        lib.qsa_probe_line_reads.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_uint32, P, I64, P]
        _PROBE = lib
    return _PROBE


def probe_time(pools, sels, hkv, row_b, steps, repeats, per_wave=64):
    """Median us per call of the bare gather over `sels` (rotating) and
    `pools` ([(k, v)] rotating, byte strides from the tensors)."""
    import ctypes
    import torch
    lib = probe_lib()
    n_max = max(int(s_.numel()) for s_ in sels)
    blocks = -(-(-(-n_max // per_wave)) // 4)
    sink = torch.zeros(blocks + 1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(i):
        k_, v_ = pools[i % len(pools)]
        s_ = sels[i % len(sels)]
        eb = k_.element_size()
        rc = lib.qsa_probe_gather(k_.data_ptr(), v_.data_ptr(), k_.stride(0) * eb, k_.stride(1) * eb, hkv,
                                  row_b, s_.data_ptr(), s_.numel(), k_.shape[0], per_wave,
                                  sink.data_ptr(), sink.numel(), stream)
        if rc != 0:
            raise RuntimeError(f"qsa_probe_gather failed ({rc})")

    for i in range(len(pools) * len(sels)):
        call(i)
    torch.cuda.synchronize()

    def run():
        for i in range(steps):
            call(i)
    return time_calls(run, steps, repeats)[0]


def gather_ceiling(args, k, v, sels, case, copies):
    """The bench's own rows (bf16 pools, its index banks) read by the bare
    gather: warm (one pool) and cold (the pool copies in turn)."""
    if probe_lib() is None:
        return None
    b = gathered_bytes(case.lengths, case.hkv)
    warm = probe_time([(k, v)], sels, case.hkv, 512, args.steps, args.repeats)
    rec = {"kernel": "qsa_probe_gather (libqsa_probe.so)", "bytes_per_call": b,
           "warm_us": round(warm, 3), "warm_GBps": round(b / (warm * 1e-6) / 1e9, 2)}
    if len(copies) > 1:
        cold = probe_time([(c_[0], c_[1]) for c_ in copies], sels, case.hkv, 512, args.steps,
                          args.repeats)
        rec.update(cold_us=round(cold, 3), cold_GBps=round(b / (cold * 1e-6) / 1e9, 2),
                   pool_copies=len(copies))
    return rec


def gather_mode(args):
    """The bare random-row gather (libqsa_probe.so) on the bench workload's
    lists: rows of 512 B (bf16), 256 B (fp8 / int8) and 128 B (int4) from
    [262144, hkv, row] pools, warm (one pool) and cold (--pool-copies pools
    in turn), for a few entries-per-wave settings.  One JSON line each."""
    import torch
    import synth
    if probe_lib() is None:
        raise SystemExit("libqsa_probe.so is not built")
    torch.cuda.set_device(0)
    case = synth.case_bs128_tp1_saturated(bs=args.bs, hkv=args.hkv)
    slots = case.k_pool.shape[0]
    sels = [torch.from_numpy(case.sel).cuda()]
    for i in range(1, args.banks):
        rng = np.random.default_rng(103_000 + i)
        sels.append(torch.from_numpy(synth.pack([synth.draw_indices(rng, n, slots)
                                                 for n in case.lengths])[0]).cuda())
    gen = torch.Generator(device="cuda").manual_seed(7)
    for row_b in (512, 256, 128):
        pools = [(torch.randint(0, 256, (slots, case.hkv, row_b), dtype=torch.uint8, device="cuda",
                                generator=gen),
                  torch.randint(0, 256, (slots, case.hkv, row_b), dtype=torch.uint8, device="cuda",
                                generator=gen)) for _ in range(max(1, args.pool_copies))]
        b = gathered_bytes(case.lengths, case.hkv, row_b)
        for per_wave in (32, 64, 128, 256):
            for variant, ps in (("warm", pools[:1]), ("cold", pools)):
                if variant == "cold" and len(pools) < 2:
                    continue
                us = probe_time(ps, sels, case.hkv, row_b, args.steps, args.repeats, per_wave)
                gbs = b / (us * 1e-6) / 1e9
                print(json.dumps({"mode": "gather", "row_bytes": row_b, "per_wave": per_wave,
                                  "variant": variant, "pool_copies": len(ps), "us_per_call": round(us, 3),
                                  "bytes_per_call": b, "GBps": round(gbs, 1),
                                  "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "workload": f"bs={case.bs} hkv={case.hkv}, 2055 uniform entries per "
                                              f"row over {slots} slots, {len(sels)} index banks"}),
                      flush=True)
        del pools
        torch.cuda.empty_cache()


LINE_POLICIES = ("plain", "non-temporal", "atomic, agent scope", "atomic, system scope")


def line_reads_mode(args):
    """Random 4-byte reads of 128-byte lines that no other read touches (the
    scale reads of a quantized pool) under each load form of
    qsa_probe_line_reads, over a 2 GiB buffer (eight times the Infinity
    Cache): us per launch and reads per second; the bytes the L2 fetches
    per read come from the TCC read-request counters of a profiled run.
    One JSON line per load form."""
    import ctypes
    import torch
    if probe_lib() is None:
        raise SystemExit("libqsa_probe.so is not built")
    torch.cuda.set_device(0)
    lib = probe_lib()
    buf_bytes = 2 << 30
    buf = torch.zeros(buf_bytes // 4, dtype=torch.float32, device="cuda")
    n_reads = 4096 * 1024
    sink = torch.zeros(n_reads // 1024, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for pol, name in enumerate(LINE_POLICIES):
        def call(i, pol=pol):
            rc = lib.qsa_probe_line_reads(buf.data_ptr(), buf_bytes, n_reads, pol, 7 + i,
                                          sink.data_ptr(), sink.numel(), stream)
            if rc != 0:
                raise RuntimeError(f"qsa_probe_line_reads failed ({rc})")
        for i in range(2):
            call(1000 + i)
        torch.cuda.synchronize()

        def run():
            for i in range(args.steps):
                call(i)
        us = time_calls(run, args.steps, args.repeats)[0]
        print(json.dumps({"mode": "line-reads", "load": name, "policy": pol, "reads": n_reads,
                          "us_per_launch": round(us, 3),
                          "Greads_per_s": round(n_reads / (us * 1e-6) / 1e9, 2),
                          "line_GBps_if_128B": round(n_reads * 128 / (us * 1e-6) / 1e9, 1),
                          "buffer_bytes": buf_bytes}), flush=True)


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


def store_mode(args):
    """qsa_kv_store throughput: `tokens` new K/V rows per call (TP1 layout,
    2 KV heads) scattered to distinct random slots of 262144-slot pools.
    Algorithmic bytes per call = reads of the bf16 rows (2 x 512 B per
    token and KV head) + slot ids + writes of codes and scales."""
    import numpy as np
    import torch
    import sparse_index_paged_amd as qsa
    import synth
    fmt = args.kv_format
    if fmt == "tiered":
        return store_tiered_mode(args)
    group = args.group or FORMATS[fmt][2]
    sdt = torch.float16 if args.scale_dtype == "f16" else torch.float32
    slots, hkv, n = 262144, args.hkv, args.tokens
    rng = np.random.default_rng(2024)
    pdt = getattr(torch, FORMATS[fmt][3])
    kc = torch.zeros((slots, hkv, FORMATS[fmt][0]), dtype=pdt, device="cuda")
    vc = torch.zeros_like(kc)
    scales = {}
    if fmt != "bf16":
        scales = dict(kv_format=fmt, group_size=group,
                      k_scale=torch.zeros((slots, hkv, 256 // group), dtype=sdt, device="cuda"),
                      v_scale=torch.zeros((slots, hkv, 256 // group), dtype=sdt, device="cuda"))
    banks = []
    for i in range(4):
        xk = synth.normal_bf16(rng, (n, hkv, 256)).cuda()
        xv = synth.normal_bf16(rng, (n, hkv, 256)).cuda()
        loc = torch.from_numpy(rng.permutation(slots)[:n].astype(np.int32)).cuda()
        banks.append((xk, xv, loc))
    for i in range(args.warmup):
        xk, xv, loc = banks[i % 4]
        qsa.kv_store(xk, xv, loc, kc, vc, **scales)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        xk, xv, loc = banks[i % 4]
        qsa.kv_store(xk, xv, loc, kc, vc, **scales)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    sb = 2 if args.scale_dtype == "f16" else 4
    b = n * 4 + n * hkv * 2 * (512 + row_bytes(fmt, group, sb))
    gbs = b / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "qsa_kv_store GB/s (bf16 rows read + codes/scales written)",
        "value": round(gbs, 2), "unit": "GB/s", "us_per_call": round(ms * 1e3, 3),
        "steps": args.steps, "warmup": args.warmup, "dtype": f"bf16 -> {fmt}",
        "config": {"workload": f"{n} tokens x {hkv} KV heads into [262144,{hkv},256] {fmt} pools "
                               f"(group {group}, {args.scale_dtype} scales)",
                   "tokens": n, "hkv": hkv, "format": fmt, "group": group,
                   "algorithmic_bytes_per_call": b},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": b, "kernel": f"qsa_store_kernel<{fmt}>"},
    }), flush=True)


def store_tiered_mode(args):
    """qsa_kv_store_tiered throughput: `tokens` new rows per call into a
    tiered pool (int4-g32 pool of 262144 slots, int8-g64 ring of ring-rows
    rows, f16 scales); slots are consecutive, as handed out in order.
    Algorithmic bytes per call = bf16 rows read + slot ids + int4 rows and
    scales written + int8 ring rows, scales and owner ids written for the
    tokens that keep a ring row."""
    import torch
    import sparse_index_paged_amd as qsa
    import synth
    slots, hkv, n, r = 262144, args.hkv, args.tokens, args.ring_rows
    rng = np.random.default_rng(2025)
    xk = synth.normal_bf16(rng, (slots, hkv, 256)).cuda()
    xv = synth.normal_bf16(rng, (slots, hkv, 256)).cuda()
    pool = qsa.TieredPool(tiered_pools(xk, xv, r))
    nb = max(1, slots // n)
    banks = [(xk[i * n:(i + 1) * n], xv[i * n:(i + 1) * n],
              torch.arange(i * n, (i + 1) * n, dtype=torch.int32, device="cuda")) for i in range(min(nb, 4))]
    for i in range(args.warmup):
        qsa.kv_store_tiered(*banks[i % len(banks)], pool)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        qsa.kv_store_tiered(*banks[i % len(banks)], pool)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kept = min(n, r)
    b = n * 4 + n * hkv * 2 * (512 + 128 + 16) + kept * (hkv * 2 * (256 + 8) + 4)
    gbs = b / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "qsa_kv_store_tiered GB/s (bf16 rows read + int4 rows and int8 ring rows written)",
        "value": round(gbs, 2), "unit": "GB/s", "us_per_call": round(ms * 1e3, 3),
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16 -> int4 + int8 ring",
        "config": {"workload": f"{n} tokens x {hkv} KV heads into a tiered pool: int4-g32 [262144,{hkv},128] "
                               f"+ int8-g64 ring of {r} rows (f16 scales), consecutive slots",
                   "tokens": n, "hkv": hkv, "ring_rows": r, "algorithmic_bytes_per_call": b,
                   "launches_per_call": 3},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": b, "kernel": "qsa_store_kernel<3> + claim + qsa_store_kernel<2>"},
    }), flush=True)


def index_mode(args):
    """qsa_index: per row the top budget / c blocks of an 8K-token (--ctx)
    context by MQA score over --index-heads heads of dim --index-dim,
    expanded to KV slots (two launches per call).  The pages give the
    indexer's context, batch sizes, budget and compression ratio but not its
    head count or width; 64 heads of dim 128 is this benchmark's choice.
    Algorithmic work per call: the block scores (hi * di multiply-adds per
    block, fp32) over the compressed keys (di bf16 + a block-table entry per
    block) and the expansion (token-table entry read + slot written per
    listed token)."""
    import torch
    import sparse_index_paged_amd as qsa
    import synth
    bs, c, budget, hi, di = args.bs, args.compress, args.budget, args.index_heads, args.index_dim
    rng = np.random.default_rng(2026)
    ctx = [args.ctx] * bs
    banks = []
    for i in range(4):
        inp = synth.index_inputs(rng, ctx, hi=hi, di=di, c=c, slots=1 << 20)
        banks.append(dict(q=inp["q"].cuda(), k=inp["k_pool"].cuda(),
                          bt=torch.from_numpy(inp["block_table"]).cuda(),
                          r2t=torch.from_numpy(inp["req_to_token"]).cuda(),
                          ctx=torch.from_numpy(inp["ctx_len"]).cuda(),
                          w=torch.from_numpy(inp["weights"]).cuda()))
    sel = torch.empty(bs * (budget + c - 1), dtype=torch.int32, device="cuda")
    cu = torch.empty(bs + 1, dtype=torch.int32, device="cuda")

    def step(i):
        d = banks[i % 4]
        qsa.index(d["q"], d["k"], d["bt"], d["r2t"], d["ctx"], budget=budget, compress_ratio=c,
                  head_weights=d["w"], sel_out=sel, cu_out=cu)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    reps = []
    for _ in range(args.repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) / args.steps)
    ms = float(np.median(reps))
    n = args.ctx // c
    listed = min(n, budget // c) * c + args.ctx % c
    # algorithmic work: the weighted query (hi * di multiply-adds per row),
    # one di-element dot product per block, and the gather of what the step
    # must read and write: the compressed keys and block-table entries of
    # every block, the queries and weights, the token-table entries and slot
    # ids of every listed token
    flops = bs * (hi * di + n * di) * 2
    byts = bs * (n * (di * 2 + 4) + listed * 8 + hi * di * 2 + hi * 4)
    gbs = byts / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "qsa_index us/call (MQA block scores + exact top-k + expansion)",
        "value": round(ms * 1e3, 3), "unit": "us/call", "higher_is_better": False,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16 in, fp32 scores",
        "timing": {"repeats": len(reps), "us_per_call_p10": round(float(np.percentile(reps, 10)) * 1e3, 3),
                   "us_per_call_p90": round(float(np.percentile(reps, 90)) * 1e3, 3)},
        "config": {"workload": f"{bs} rows x {args.ctx}-token contexts, compress ratio {c}, budget {budget} "
                               f"({budget + c - 1}-entry rows), {hi} index heads of dim {di}",
                   "bs": bs, "ctx": args.ctx, "compress_ratio": c, "budget": budget,
                   "index_heads": hi, "index_dim": di, "launches_per_call": 2,
                   "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": byts},
        # the step reads each compressed key once and does di multiply-adds
        # per block: an HBM-side gather, far below both the HBM and the fp32
        # roofline at these sizes -- both kernels are bound by latency chains
        # (score: block table -> key rows -> dot products; select: radix
        # passes separated by workgroup barriers)
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 4),
                     "kernel": "qsa_index_score_kernel + qsa_index_select_kernel"},
    }), flush=True)


def time_calls(run_steps, calls: int, repeats: int):
    """`repeats` runs of run_steps() (which issues `calls` decode calls on
    torch's current stream), each bracketed by HIP events on that stream;
    returns (median, p10, p90) in microseconds per call."""
    import torch
    stream = torch.cuda.current_stream()
    per_call = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        run_steps()
        e1.record(stream)
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / calls)
    return (float(np.median(per_call)), float(np.percentile(per_call, 10)),
            float(np.percentile(per_call, 90)))


def configs_mode(args):
    """One JSON line per workload of the five measured configurations:
    bs=1 TP1 L=128 over a 4096-slot pool; bs=16 TP2 with mixed lengths over
    65536 slots; bs=128 TP1 saturated (the default line's workload); bs=64
    TP1 quantized pools (fp8 + f32 row scale, int8 + f32 row scale, int4 +
    f32 scale per 32 channels) over 131072 slots with L~U[256,2055], warm
    (one pool) and cold (4 pool copies rotating, 4 x the Infinity Cache's
    256 MB is not reached by one copy); and the graph-replay sweep (TP1 and
    TP2, every bs 1..16 plus 17/24/32/48/64/96/128, short / medium /
    saturated lists with duplicate runs), timed as (a) a captured graph of 8
    calls over 8 resident index banks and (b) per replay of one captured
    call with its cu_seqlens and indices rewritten on the device before it.
    Every configuration's eager timing runs before any graph is captured.
    --only selects configurations by substrings of their names."""
    import torch

    import sparse_index_paged_amd as qsa
    import synth

    torch.cuda.set_device(0)
    qsa.workspace_reserve(128, 24, 2)
    steps, reps = args.steps, args.repeats

    def log(msg):
        print(f"[configs] {msg}", file=sys.stderr, flush=True)

    def emit(name, workload, b_kv, us, extra=None):
        med, p10, p90 = us
        gbs = b_kv / (med * 1e-6) / 1e9
        rec = {"mode": "configs", "config": name, "workload": workload,
               "us_per_call": round(med, 3), "us_p10": round(p10, 3), "us_p90": round(p90, 3),
               "gathered_kv_bytes_per_call": int(b_kv), "GBps": round(gbs, 1),
               "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if extra:
            rec.update(extra)
        print(json.dumps(rec), flush=True)

    def bank_sel(seed, lengths, slots):
        """Another packed index list for the same lengths: one generator
        per bank, every row its own draws."""
        rng = np.random.default_rng(seed)
        return synth.pack([synth.draw_indices(rng, n, slots) for n in lengths])[0]

    def eager_us(call):
        def run():
            for i in range(steps):
                call(i)
        run()
        return time_calls(run, steps, reps)

    def graph_us(call):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(8):
                call(i)
        g.replay()
        n8 = max(1, steps // 8)

        def run8():
            for _ in range(n8):
                g.replay()
        med, p10, p90 = time_calls(run8, 8 * n8, reps)
        del g
        return {"graph_us_per_call": round(med, 3), "graph_us_p10": round(p10, 3),
                "graph_us_p90": round(p90, 3)}

    # Every configuration is set up first and timed eagerly (the figure that
    # matches the default line), then replayed from captured graphs: once a
    # graph has been captured and replayed in a process, later eager launches
    # of the same kernel run about 3 us slower per call on this stack.
    jobs = []  # (name, workload, gathered bytes, call(i), extra fields)
    keep = []  # device tensors the calls use

    def bf16_job(case, bank_seed, name, workload):
        slots = case.k_pool.shape[0]
        sels = [case.sel] + [bank_sel(bank_seed + i, case.lengths, slots) for i in range(1, 4)]
        q, k, v = case.q.cuda(), case.k_pool.cuda(), case.v_pool.cuda()
        cu = torch.from_numpy(case.cu).cuda()
        sd = [torch.from_numpy(s).cuda() for s in sels]
        out = torch.empty(case.bs, case.hq, 256, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(case.bs, case.hq, dtype=torch.float32, device="cuda")

        pool = qsa.KvPool(k, v)

        def call(i):
            pool.decode(q, sd[i % 4], cu, out=out, lse=lse)
        jobs.append((name, workload, gathered_bytes(case.lengths, case.hkv), call,
                     {"splits": qsa.plan(case.bs, case.hkv)[0]}))
        keep.append((q, k, v, cu, sd, out, lse))
        return k, v

    only = [o for o in (args.only or "").split(",") if o]

    def want(name):
        return not only or any(o in name for o in only)

    k_big = v_big = None
    if want("bs1_tp1_L128"):
        bf16_job(synth.case_bs1_tp1(), 101_000, "bs1_tp1_L128",
                 "bs=1 TP1 (24Q/2KV) bf16 pools [4096,2,256], 128 uniform indices")
    if want("bs16_tp2_mixed"):
        bf16_job(synth.case_bs16_tp2_mixed(), 102_000, "bs16_tp2_mixed",
                 "bs=16 TP2 (12Q/1KV) bf16 pools [65536,1,256], 8 rows L~U[1,64], 4 rows 2055, "
                 "4 rows L~U[65,2054]")
    if want("bs128_tp1_saturated"):
        k_big, v_big = bf16_job(synth.case_bs128_tp1_saturated(), 103_000, "bs128_tp1_saturated",
                                "bs=128 TP1 (24Q/2KV) bf16 pools [262144,2,256], 2055 entries per "
                                "row, 5% keys x8")

    # ---- quantized pools, warm (one pool) and cold (4 copies rotating)
    for fmt, group, seed in (("fp8", 256, 1041), ("int8", 256, 1042), ("int4", 32, 1043)):
        if not want(f"bs64_tp1_{fmt}_warm") and not want(f"bs64_tp1_{fmt}_cold"):
            continue
        log(f"bs=64 TP1 {fmt}: pools")
        case = synth.case_bs64_tp1_quantsrc(seed)
        kc, vc, ks, vs = quantized_pools(case.k_pool.cuda(), case.v_pool.cuda(), fmt, group,
                                         torch.float32)
        copies = [(kc, vc, ks, vs)] + [tuple(t.clone() for t in (kc, vc, ks, vs)) for _ in range(3)]
        slots = case.k_pool.shape[0]
        sels = [case.sel] + [bank_sel(seed * 1000 + i, case.lengths, slots) for i in range(1, 4)]
        q = case.q.cuda()
        cu = torch.from_numpy(case.cu).cuda()
        sd = [torch.from_numpy(s).cuda() for s in sels]
        out = torch.empty(case.bs, case.hq, 256, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(case.bs, case.hq, dtype=torch.float32, device="cuda")
        keep.append((copies, q, cu, sd, out, lse))
        b_kv = gathered_bytes(case.lengths, case.hkv, row_bytes(fmt, group, 4))
        pools = [qsa.KvPool(k_, v_, kv_format=fmt, k_scale=ks_, v_scale=vs_, group_size=group)
                 for k_, v_, ks_, vs_ in copies]
        keep.append(pools)
        for variant, ncopy in (("warm", 1), ("cold", 4)):
            def call(i, ncopy=ncopy, pools=pools, q=q, cu=cu, sd=sd, out=out, lse=lse):
                pools[i % ncopy].decode(q, sd[i % 4], cu, out=out, lse=lse)
            jobs.append((f"bs64_tp1_{fmt}_{variant}",
                         f"bs=64 TP1 (24Q/2KV) {fmt} pools [131072,2,{FORMATS[fmt][0]}] + f32 scales "
                         f"per {group} channels (written by qsa_kv_store), L~U[256,2055], "
                         f"{ncopy} pool cop{'y' if ncopy == 1 else 'ies'} rotating", b_kv, call,
                         {"kv_format": fmt, "group": group, "pool_copies": ncopy}))

    eager = []
    for name, _, _, call, _ in jobs:
        log(f"{name}: eager")
        eager.append(eager_us(call))
    for (name, workload, b_kv, call, extra), us in zip(jobs, eager):
        log(f"{name}: graph")
        emit(name, workload, b_kv, us, {**extra, **graph_us(call)})
    del keep, jobs
    torch.cuda.empty_cache()

    # ---- graph-replay sweep over the bench's bf16 pools (TP2 uses KV head 0)
    if not want("graph_sweep"):
        return
    if k_big is None:
        case = synth.case_bs128_tp1_saturated()
        k_big, v_big = case.k_pool.cuda(), case.v_pool.cuda()
    slots = k_big.shape[0]
    for hkv in (2, 1):
        kd, vd = (k_big, v_big) if hkv == 2 else (k_big[:, :1], v_big[:, :1])
        hq = 12 * hkv
        for kind in ("short", "medium", "saturated"):
            log(f"graph sweep hkv={hkv} {kind}")
            table = {}
            for bs in synth.SWEEP_BS:
                banks = synth.sweep_bank(1050 + bs, bs, kind, slots, banks=8)
                sel_banks = [torch.from_numpy(s).cuda() for s, _ in banks]
                cu_banks = [torch.from_numpy(c).cuda() for _, c in banks]
                q = synth.normal_bf16(np.random.default_rng(bs * 7 + hkv), (bs, hq, 256)).cuda()
                out = torch.empty(bs, hq, 256, dtype=torch.bfloat16, device="cuda")
                lse = torch.empty(bs, hq, dtype=torch.float32, device="cuda")
                qsa.decode(q, kd, vd, sel_banks[0], cu_banks[0], out=out, lse=lse)
                torch.cuda.synchronize()
                g8 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g8):
                    for b in range(8):
                        qsa.decode(q, kd, vd, sel_banks[b], cu_banks[b], out=out, lse=lse)
                g8.replay()
                n8 = max(1, steps // 8)

                def run8():
                    for _ in range(n8):
                        g8.replay()
                us8 = time_calls(run8, 8 * n8, reps)[0]
                sel_buf, cu_buf = sel_banks[0].clone(), cu_banks[0].clone()
                g1 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g1):
                    qsa.decode(q, kd, vd, sel_buf, cu_buf, out=out, lse=lse)
                g1.replay()

                def run1():
                    for r in range(steps):
                        sel_buf.copy_(sel_banks[r % 8])
                        cu_buf.copy_(cu_banks[r % 8])
                        g1.replay()
                us1 = time_calls(run1, steps, reps)[0]
                mean_b = float(np.mean([gathered_bytes(np.diff(c), hkv) for _, c in banks]))
                table[str(bs)] = {"us_per_call": round(us8, 2),
                                  "GBps": round(mean_b / (us8 * 1e-6) / 1e9, 1),
                                  "us_per_replay_with_rewrite": round(us1, 2)}
                del g8, g1
            print(json.dumps({"mode": "configs", "config": f"graph_sweep_{'tp1' if hkv == 2 else 'tp2'}_{kind}",
                              "workload": f"{'TP1 (24Q/2KV)' if hkv == 2 else 'TP2 (12Q/1KV)'} bf16 pools "
                                          f"[262144,{hkv},256], {kind} lists with duplicate runs, "
                                          "8 banks per bs",
                              "counters_at_rest": all(c == 0 for c in qsa.debug_counters()),
                              "by_bs": table}), flush=True)


def phases_mode(args):
    """Per-workgroup phase breakdown of decode calls, from the phase stamps
    of the measurement build libqsa_stamps.so (include/qsa_stamps.h): the
    bench workload's lists at --bs / --hkv over bf16 pools, --warmup calls
    without stamps, then --steps stamped calls.  For each stamped call the
    median and the slowest workgroup of every phase; the line reports the
    medians of those over the calls, in us (stamps tick at 100 MHz)."""
    import torch
    import synth
    from sparse_index_paged_amd import _binding as B
    lib = B.load_stamps_library()
    torch.cuda.set_device(0)
    case = synth.case_bs128_tp1_saturated(bs=args.bs, hkv=args.hkv)
    slots = case.k_pool.shape[0]
    sels = [case.sel]
    for i in range(1, 4):
        rng = np.random.default_rng(103_000 + i)
        sels.append(synth.pack([synth.draw_indices(rng, n, slots) for n in case.lengths])[0])
    q, k, v = case.q.cuda(), case.k_pool.cuda(), case.v_pool.cuda()
    cu = torch.from_numpy(case.cu).cuda()
    sd = [torch.from_numpy(s_).cuda() for s_ in sels]
    out = torch.empty(case.bs, case.hq, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.bs, case.hq, dtype=torch.float32, device="cuda")
    ns, nw = ctypes.c_int(), ctypes.c_int()
    if lib.qsa_plan(case.bs, case.hkv, ctypes.byref(ns), ctypes.byref(nw)) != 0:
        raise RuntimeError(lib.qsa_last_error().decode())
    stamps = torch.zeros(nw.value * 8, dtype=torch.int64, device="cuda")
    qd, kd, vd = B.describe(q), B.describe(k), B.describe(v)
    cd, od, ld = B.describe(cu), B.describe(out), B.describe(lse)
    sdd = [B.describe(x) for x in sd]
    stream = B._stream_handle(None)

    def call(i, stamped):
        lib.qsa_debug_set_phase_stamps(stamps.data_ptr() if stamped else None,
                                       stamps.numel() if stamped else 0)
        if lib.qsa_decode(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), None,
                          ctypes.byref(sdd[i % 4]), ctypes.byref(cd), ctypes.byref(od),
                          ctypes.byref(ld), stream) != 0:
            raise RuntimeError(lib.qsa_last_error().decode())

    for i in range(args.warmup):
        call(i, False)
    torch.cuda.synchronize()
    keys = ("start_skew", "cu_seqlens", "first_rows", "loop", "wave_merge", "arrival",
            "last_split_merge", "end")
    per_call = {k_: [] for k_ in keys}
    spans = []
    for i in range(args.steps):
        stamps.zero_()
        call(i, True)
        torch.cuda.synchronize()
        st = stamps.view(nw.value, 8).cpu().numpy().astype(np.float64) * 0.01  # us
        act = st[:, 1] > 0
        s_ = st[act]
        t0 = st[st[:, 0] > 0, 0].min()
        end = np.where(s_[:, 6] > 0, s_[:, 6], s_[:, 5])
        split = s_[:, 5] > 0
        last = split & (s_[:, 6] > 0)
        tiled = s_[:, 2] > 0
        ph = {"start_skew": s_[:, 0] - t0, "cu_seqlens": s_[:, 1] - s_[:, 0],
              "first_rows": s_[tiled, 2] - s_[tiled, 1], "loop": s_[tiled, 3] - s_[tiled, 2],
              "wave_merge": s_[:, 4] - s_[:, 3], "arrival": (s_[split, 5] - s_[split, 4]),
              "last_split_merge": (s_[last, 6] - s_[last, 5]), "end": end - t0}
        for k_ in keys:
            x = ph[k_]
            per_call[k_].append((float(np.median(x)), float(np.max(x))) if x.size else (0.0, 0.0))
        spans.append(float(end.max() - t0))
    rec = {"mode": "phases", "bs": case.bs, "hkv": case.hkv, "splits": ns.value, "workgroups": nw.value,
           "stamped_calls": args.steps,
           "span_us": round(float(np.median(spans)), 2),
           "phases_us": {k_: {"median_wg": round(float(np.median([a for a, _ in v_])), 2),
                              "slowest_wg": round(float(np.median([b_ for _, b_ in v_])), 2)}
                         for k_, v_ in per_call.items()},
           "workload": f"bench lists at bs={case.bs} hkv={case.hkv} (2055 entries per row), bf16 pools "
                       f"[262144,{case.hkv},256], libqsa_stamps.so"}
    print(json.dumps(rec), flush=True)


def splits_mode(args):
    """Every forced split count (1-12 and 16) at each --sweep-bs batch size,
    both layouts, over the bench workload's lists (4 rotating banks), eager:
    one JSON line per (layout, bs) with the time of each count, the plan's
    count and what the plan loses against the fastest measured count."""
    import torch
    import sparse_index_paged_amd as qsa
    import synth
    torch.cuda.set_device(0)
    case = synth.case_bs128_tp1_saturated()
    slots = case.k_pool.shape[0]
    sels = [case.sel]
    for i in range(1, 4):
        rng = np.random.default_rng(103_000 + i)
        sels.append(synth.pack([synth.draw_indices(rng, n, slots) for n in case.lengths])[0])
    q, k, v = case.q.cuda(), case.k_pool.cuda(), case.v_pool.cuda()
    cu = torch.from_numpy(case.cu).cuda()
    sd = [torch.from_numpy(s_).cuda() for s_ in sels]
    qsa.workspace_reserve(128, 24, 2)
    counts = list(range(1, 13)) + [16]
    for hkv in (2, 1):
        pool = qsa.KvPool(k, v) if hkv == 2 else qsa.KvPool(k[:, :1], v[:, :1])
        for bs in (int(x) for x in args.sweep_bs.split(",") if x):
            hq = 12 * hkv
            qq, cub = q[:bs, :hq].contiguous(), cu[:bs + 1].contiguous()
            out = torch.empty(bs, hq, 256, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(bs, hq, dtype=torch.float32, device="cuda")
            qsa.set_option("splits", 0)
            plan = qsa.plan(bs, hkv)[0]
            us = {}
            try:
                for n in counts:
                    qsa.set_option("splits", n)

                    def run():
                        for i in range(100):
                            pool.decode(qq, sd[i % 4], cub, out=out, lse=lse)
                    run()
                    us[n] = round(time_calls(run, 100, 3)[0], 3)
            finally:
                qsa.set_option("splits", 0)
            best = min(us, key=us.get)
            print(json.dumps({"mode": "splits", "layout": "TP1" if hkv == 2 else "TP2", "bs": bs,
                              "plan": plan, "us_by_splits": us, "fastest": best,
                              "plan_loss_us": round(us[plan] - us[best], 3) if plan in us else None,
                              "workload": "bf16 pools [262144, Hkv, 256], 2055 uniform entries per row, "
                                          "4 rotating index banks, 100 eager calls x 3 repeats"}),
                  flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats of --steps launches")
    ap.add_argument("--timing", choices=["eager", "graph"], default="eager",
                    help="time the steps as eager launches (default) or as a replayed HIP graph")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--banks", type=int, default=4)
    ap.add_argument("--bs", type=int, default=128)
    ap.add_argument("--hkv", type=int, default=2, choices=[1, 2])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-copy reference rate")
    ap.add_argument("--mode", choices=["decode", "copy", "store", "index", "configs", "gather", "line-reads", "splits",
                                       "phases"],
                    default="decode")
    ap.add_argument("--ctx", type=int, default=8192, help="index mode: context tokens per row")
    ap.add_argument("--compress", type=int, default=4, help="index mode: compression ratio")
    ap.add_argument("--budget", type=int, default=2048, help="index mode: token budget")
    ap.add_argument("--index-heads", type=int, default=64)
    ap.add_argument("--index-dim", type=int, default=128)
    ap.add_argument("--kv-format", choices=list(FORMATS) + ["tiered"], default="bf16")
    ap.add_argument("--ring-rows", type=int, default=8192, help="tiered: ring rows (power of two)")
    ap.add_argument("--hot-frac", type=float, default=None,
                    help="tiered: fraction of entries drawn from the ring's slots")
    ap.add_argument("--group", type=int, default=None)
    ap.add_argument("--scale-dtype", choices=["f32", "f16"], default="f32")
    ap.add_argument("--tokens", type=int, default=32768, help="tokens per store call")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--split-target", type=int, default=None)
    ap.add_argument("--splits", type=int, default=None, help="force this many splits per (row, KV head)")
    ap.add_argument("--min-split-keys", type=int, default=None)
    ap.add_argument("--waves", type=int, default=None)
    ap.add_argument("--pool-copies", type=int, default=4,
                    help="decode: also time the calls over this many pool copies in turn (cold); "
                         "0 or 1 skips it")
    ap.add_argument("--cold", action="store_true",
                    help="decode: every timed step (warm-up included) uses the pool copies in turn, "
                         "so the reported value is the cold rate")
    ap.add_argument("--no-graph", action="store_true", help="decode: skip the graph-replay timing")
    ap.add_argument("--no-probe", action="store_true", help="decode: skip the bare-gather ceiling")
    ap.add_argument("--only", default=None,
                    help="configs mode: comma-separated substrings of the configuration names to run")
    ap.add_argument("--pool-layout", choices=["slot-major", "head-major"], default="slot-major",
                    help="decode, bf16: pools stored [slots][Hkv][256] (the pages' layout) or each KV "
                         "head's rows contiguous, passed as the same [slots, Hkv, 256] view by strides")
    ap.add_argument("--sweep-bs", default="1,2,3,4,6,8,12,16,20,24,28,32,40,48,56,64,72,80,96,112,128",
                    help="splits mode: batch sizes")
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
    if args.mode == "store":
        store_mode(args)
        return
    if args.mode == "index":
        index_mode(args)
        return
    if args.mode == "configs":
        configs_mode(args)
        return
    if args.mode == "line-reads":
        return line_reads_mode(args)
    if args.mode == "gather":
        gather_mode(args)
        return
    if args.mode == "splits":
        splits_mode(args)
        return
    if args.mode == "phases":
        phases_mode(args)
        return

    import numpy as np

    import sparse_index_paged_amd as qsa
    import synth

    if args.split_target:
        qsa.set_option("split_target", args.split_target)
    if args.splits:
        qsa.set_option("splits", args.splits)
    if args.min_split_keys:
        qsa.set_option("min_split_keys", args.min_split_keys)
    if args.waves:
        qsa.set_option("waves_per_workgroup", args.waves)

    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    case = synth.case_bs128_tp1_saturated(bs=args.bs, hkv=args.hkv)
    slots = case.k_pool.shape[0]
    bank_sels = [case.sel]
    for i in range(1, args.banks):
        rng = np.random.default_rng(103_000 + i)
        lists = [synth.draw_indices(rng, n, slots) for n in case.lengths]
        bank_sels.append(synth.pack(lists)[0])
    if args.kv_format == "tiered" and args.hot_frac is not None:
        recent = np.arange(slots - args.ring_rows, slots)
        bank_sels = [synth.tiered_lists(np.random.default_rng(104_000 + i), case.lengths, slots,
                                        recent, args.hot_frac)[0] for i in range(args.banks)]
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)

    q = case.q.cuda()
    k = case.k_pool.cuda()
    v = case.v_pool.cuda()
    fmt = args.kv_format
    if args.pool_layout == "head-major":
        if fmt != "bf16":
            raise SystemExit("--pool-layout head-major applies to bf16 pools")
        k = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
        v = v.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    group = args.group or FORMATS.get(fmt, (0, 0, 32))[2]
    sdt = torch.float16 if args.scale_dtype == "f16" else torch.float32
    qkw = {}
    tiered = None
    if fmt == "tiered":
        tiered_arrays = tiered_pools(k, v, args.ring_rows)
        del k, v
        owner_host = tiered_arrays["owner"].cpu().numpy()
        tiered = qsa.TieredPool(tiered_arrays)  # descriptor built once for every call
    elif fmt != "bf16":
        kc, vc, ks, vs = quantized_pools(k, v, fmt, group, sdt)
        del k, v
        k, v = kc, vc
        qkw = dict(kv_format=fmt, k_scale=ks, v_scale=vs, group_size=group)
    cu = torch.from_numpy(case.cu).cuda()
    sels = [torch.from_numpy(s).cuda() for s in bank_sels]
    out = torch.empty(case.bs, case.hq, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.bs, case.hq, dtype=torch.float32, device="cuda")
    qsa.workspace_reserve(case.bs, case.hq, case.hkv)
    torch.cuda.synchronize()

    # pool copies for the cold timing (a model's layers each have their own
    # pool, so consecutive calls read different pools); with --cold every
    # timed step, warm-up included, uses them in turn
    copies = []
    if args.pool_copies > 1 and tiered is None:
        base = (k, v, qkw.get("k_scale"), qkw.get("v_scale"))
        copies = [base] + [tuple(None if t is None else t.clone() for t in base)
                           for _ in range(args.pool_copies - 1)]
        torch.cuda.synchronize()
    if args.cold and not copies:
        raise SystemExit("--cold needs --pool-copies >= 2 and a single-tier pool")

    # every pool (and pool copy) is passed as a KvPool, whose descriptors are
    # built once, as a serving loop over persistent pools would
    fkw = {key: val for key, val in qkw.items() if key in ("kv_format", "group_size")}
    copy_pools = [qsa.KvPool(kk, vv, k_scale=ks_, v_scale=vs_, **fkw) for kk, vv, ks_, vs_ in copies]

    def cold_step(i):
        copy_pools[i % len(copy_pools)].decode(q, sels[i % len(sels)], cu, out=out, lse=lse)

    if tiered is not None:
        def step(i):
            qsa.decode_tiered(q, tiered, sels[i % len(sels)], cu, out=out, lse=lse)
    elif args.cold:
        step = cold_step
    else:
        kv_pool = qsa.KvPool(k, v, **qkw)

        def step(i):
            kv_pool.decode(q, sels[i % len(sels)], cu, out=out, lse=lse)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(run_steps):
        """`repeats` timed runs of `steps` calls, each bracketed by HIP
        events on the stream the kernels run on; ms per call of each."""
        stream = torch.cuda.current_stream()
        out_ms = []
        for _ in range(args.repeats):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            run_steps()
            end.record(stream)
            torch.cuda.synchronize()
            out_ms.append(start.elapsed_time(end) / args.steps)
        return out_ms

    def eager_steps():
        for i in range(args.steps):
            step(i)

    # eager timing (reported); with --timing graph the `steps` calls (index
    # banks rotating as in the eager loop) are also captured once into a HIP
    # graph and replayed, and that timing is reported instead
    eager_ms = timed(eager_steps)
    warm_us = float(np.median(eager_ms)) * 1e3

    # cold: the same calls over the pool copies in turn, so that the
    # Infinity Cache cannot hold what a call re-reads from the previous ones
    cold = None
    if copies:
        if args.cold:
            cold_ms = eager_ms
        else:
            def cold_steps():
                for i in range(args.steps):
                    cold_step(i)
            cold_steps()
            cold_ms = timed(cold_steps)
        cold = {"us_per_call": round(float(np.median(cold_ms)) * 1e3, 3),
                "us_p10": round(float(np.percentile(cold_ms, 10)) * 1e3, 3),
                "us_p90": round(float(np.percentile(cold_ms, 90)) * 1e3, 3),
                "pool_copies": len(copies),
                "pool_bytes_rotated": int(sum(t.numel() * t.element_size() for c_ in copies
                                              for t in c_ if t is not None))}

    # bare-gather ceiling (libqsa_probe.so): the same rows, nothing computed
    probe = gather_ceiling(args, k, v, sels, case, copies) if (
        fmt == "bf16" and not args.no_probe) else None

    # graph replay of the same steps (after every eager timing: once a graph
    # has been captured in a process, later eager launches run slower)
    graph_ms = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_steps()
        graph.replay()
        torch.cuda.synchronize()
        graph_ms = timed(graph.replay)
        del graph
    reps_ms = eager_ms
    timing_mode = "eager, pool copies in turn (cold)" if args.cold else "eager"
    if args.timing == "graph":
        reps_ms = graph_ms
        timing_mode = "graph"
    ms_per_step = float(np.median(reps_ms))
    counters_ok = all(c == 0 for c in qsa.debug_counters())

    hot_share = None
    if tiered is not None:
        per_bank = [tiered_gathered_bytes(s_, case.cu, owner_host, case.hkv) for s_ in bank_sels]
        b_kv = int(sum(b for b, _ in per_bank) / len(per_bank))
        hot_share = round(sum(h for _, h in per_bank) / len(per_bank), 4)
    else:
        rb = row_bytes(fmt, group, 2 if args.scale_dtype == "f16" else 4)
        b_kv = gathered_bytes(case.lengths, case.hkv, rb)
    gbs = b_kv / (ms_per_step * 1e-3) / 1e9
    splits, wgs = qsa.plan(case.bs, case.hkv)
    traffic = committed_traffic() if fmt == "bf16" else None
    if fmt == "bf16":
        pool_desc = "bf16 pools"
    elif tiered is not None:
        pool_desc = (f"tiered pool (int4-g32 + int8-g64 ring of {args.ring_rows} rows holding the "
                     f"last written slots, f16 scales, written by qsa_kv_store_tiered; "
                     f"{hot_share:.1%} of entries read the ring)")
    else:
        pool_desc = f"{fmt} pools (group {group}, {args.scale_dtype} scales, written by qsa_kv_store)"
    if cold is not None:
        cg = b_kv / (cold["us_per_call"] * 1e-6) / 1e9
        cold.update(GBps=round(cg, 2), frac=round(cg / HBM_PEAK_GBS, 4))

    timing = {"mode": timing_mode, "repeats": len(reps_ms), "steps_per_repeat": args.steps,
              "us_per_call_eager_median": round(warm_us, 3),
              "us_per_call_p10": round(float(np.percentile(reps_ms, 10)) * 1e3, 3),
              "us_per_call_median": round(ms_per_step * 1e3, 3),
              "us_per_call_p90": round(float(np.percentile(reps_ms, 90)) * 1e3, 3)}
    if graph_ms is not None:
        timing["us_per_call_graph_median"] = round(float(np.median(graph_ms)) * 1e3, 3)
        timing["graph_GBps"] = round(b_kv / (float(np.median(graph_ms)) * 1e-3) / 1e9, 2)
    # the bf16 path is bound by the gather (committed counters: traffic equal
    # to the algorithmic bytes, MFMA busy a few percent); the quantized and
    # tiered paths are bound by per-tile work, not established as a single
    # unit's roofline
    bound = "hbm" if fmt == "bf16" else None
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(ms_per_step * 1e3, 3),
        "timing": timing,
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if fmt == "bf16" else f"bf16 ({fmt} pools)",
        "data": "synthetic",
        "config": {
            "workload": f"packed QSA decode bs={case.bs} "
                        f"{'TP1 (24Q/2KV' if case.hkv == 2 else 'TP2 (12Q/1KV'}, D=256) {pool_desc} "
                        f"[262144,{case.hkv},256], 2055 selected slots per row, 5% keys x8",
            "bs": case.bs, "hq": case.hq, "hkv": case.hkv, "head_dim": 256,
            "sel_per_row": int(case.lengths.max()), "pool_slots": int(case.k_pool.shape[0]),
            "index_banks": len(sels), "splits": splits, "workgroups": wgs,
            "pool_copies_timed": len(copies) if args.cold else 1,
            **({"ring_rows": args.ring_rows, "hot_share": hot_share} if tiered is not None else {}),
            **({"pool_layout": "head-major"} if args.pool_layout == "head-major" else {}),
            "gathered_kv_bytes_per_call": b_kv, "counters_at_rest": counters_ok,
        },
        "roofline": {
            "bound": bound,
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (f"{os.path.relpath(TRAFFIC_FILE, ROOT)} (rocprofv3 --pmc FETCH_SIZE / "
                               f"WRITE_SIZE, copy-calibrated) for kernel source sha {kernel_sha()}"
                               if traffic is not None else None),
            "mfma_busy_pct": committed_mfma_busy() if fmt == "bf16" else None,
            "mfma_busy_source": (f"{os.path.relpath(COUNTERS_FILE, ROOT)} for kernel source sha "
                                 f"{kernel_sha()}" if fmt == "bf16" and committed_mfma_busy() is not None
                                 else None),
            "algorithmic_bytes_per_launch": b_kv,
            "kernel": f"qsa_decode_kernel<{fmt}>",
            "cold": cold,
            "gather_ceiling": probe,
        },
        "cpu_baseline": None,
    }
    if probe is not None:
        line["roofline"]["frac_of_gather_ceiling"] = round(gbs / probe["warm_GBps"], 4)
        if cold is not None and probe.get("cold_GBps"):
            cold["frac_of_gather_ceiling"] = round(cold["GBps"] / probe["cold_GBps"], 4)
    if not args.no_copy:
        cr = copy_rate()
        line["roofline"]["copy_GBps"] = round(cr, 1)
        line["roofline"]["frac_of_copy"] = round(gbs / cr, 4)
    if not args.no_cpu_baseline and fmt == "bf16":
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
