"""Benchmark of the exact-attention hot path on one MI355X.

One step = one causal prefill of 28 query heads / 4 KV heads, N = 16,384, d = 128
(bf16 in, fp32 accumulation, O bf16 + LSE fp32) followed by one split-KV decode of a
single query token against a contiguous 32,768-token bf16 cache (28/4 heads, 64
chunks of 512 tokens, then the LSE combine).  Inputs are seeded synthetic N(0,1)
values already resident in HBM.  The decode reads one of 8 distinct cache copies
per step (512 MiB in total, twice the Infinity Cache) so its bytes come from HBM.

Prints one JSON line.  `value` is the prefill throughput in TFLOP/s (algorithmic
FLOPs 2*B*Hq*d*N^2 per launch, i.e. the causal half of the dense 4*B*Hq*d*N^2);
the decode figure (HBM GB/s over K+V read once plus q and o) is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak (published)
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (published)
METRIC = "causal prefill TFLOP/s (N=16k, d=128) + split-KV decode HBM GB/s at 32k"
CSRC = os.path.join(ROOT, "exact_io_aware_prefill_amd", "csrc")
# HBM traffic per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script,
# valid while the kernel source they were taken on is unchanged (sha256 recorded)
TRAFFIC = {
    "prefill": {"file": os.path.join(ROOT, "profiles", "prefill_bf16_n16384_traffic.json"),
                "src": os.path.join(CSRC, "prefill_bf16.hip"), "kernel": "prefill_bf16_kernel<128, false, 1, 3>"},
    "decode": {"file": os.path.join(ROOT, "profiles", "decode_split_s32768_traffic.json"),
               "src": os.path.join(CSRC, "decode.hip"), "kernel": "decode_split_kernel<128, false, false, false, false>",
               # the 32k decode's dispatches only (256 workgroups of 512 threads), not the
               # paged batch's, which run the same kernel on a larger grid
               "grid": 256 * 512},
    "paged": {"file": os.path.join(ROOT, "profiles", "decode_split_paged_b32_traffic.json"),
              "src": os.path.join(CSRC, "decode.hip"), "kernel": "decode_split_kernel<128, false, false, false, true>"},
    "fp8": {"file": os.path.join(ROOT, "profiles", "prefill_fp8_n16384_traffic.json"),
            "src": os.path.join(CSRC, "prefill_fp8.hip"), "kernel": "prefill_fp8_kernel<128, false, false>"},
}
COPY_BYTES = 1 << 30  # reference dispatch for the counters: a 1 GiB device-to-device copy
READ_GRIDS = (256, 512, 1024, 2048, 4096, 8192)  # workgroup counts of the floor's read sweep
BALANCED_WORKGROUPS = 256  # the decode's balanced split: workgroups in all (include/attn.h, attn_decode)
N_KV_COPIES = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle leg")
    ap.add_argument("--only", choices=["prefill", "decode", "fp8"], default=None,
                    help="time one part only (profiling runs)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 prefill measurement")
    ap.add_argument("--no-paged", action="store_true", help="skip the batched paged decode measurement")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed launches of the leg's own kernel, for about this long, before each prefill "
                         "leg's warm-up (0: none)")
    ap.add_argument("--prefill-sweep", action="store_true",
                    help="time only the causal prefill of the short and long prompt workloads (N = 2048, 8192, "
                         "16384, 30720; 28/4 heads, d = 128), print one JSON line and exit (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference dispatch for HBM counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/*_traffic.json from two rocprofv3 counter runs, then exit")
    ap.add_argument("--traffic-command", default="", help="command recorded with --write-traffic")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the fp64 oracle on every workload (host CPU only, no GPU) and print one JSON line")
    ap.add_argument("--oracle-configs", default="c1,c2,c3-8192,c3-16384,c3-30720,c4,c5",
                    help="workloads timed by --oracle-table")
    ap.add_argument("--oracle-threads", type=int, default=0,
                    help="OpenMP threads of the oracle in --oracle-table (0: the runtime's default)")
    ap.add_argument("--oracle-budget", type=float, default=10.0,
                    help="approximate seconds of oracle work per sampled workload in --oracle-table")
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(which: str):
    """HBM bytes per launch of the named kernel from committed counter runs, if they
    still describe the current kernel source; else None."""
    t = TRAFFIC[which]
    try:
        with open(t["file"]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_hash(t["src"]):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(csv_path: str, counter: str):
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def write_traffic(fetch_csv: str, write_csv: str, command: str):
    """Turn two counter runs of this script (FETCH_SIZE, then WRITE_SIZE; each with
    --copy-calibration) into per-launch HBM byte records for the prefill and decode
    split kernels.  Counter values are KiB per dispatch; each counter is scaled by
    the factor that makes it read COPY_BYTES for the 1 GiB copy dispatch."""
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, name)
        copy_kib = max(v for k, _, v in rows if "copyBuffer" in k)  # the 1 GiB copy is the largest
        factor = COPY_BYTES / (copy_kib * 1024.0)
        for which, t in TRAFFIC.items():
            vals = [v for k, g, v in rows if t["kernel"] in k and t.get("grid") in (None, g)]
            if not vals:
                continue
            rec = out.setdefault(which, {"calibration": {}})
            rec[name.lower() + "_kib_avg"] = sum(vals) / len(vals)
            rec[name.lower() + "_dispatches"] = len(vals)
            rec[name.lower() + "_bytes"] = sum(vals) / len(vals) * 1024.0 * factor
            rec["calibration"][name] = {"copy_bytes": COPY_BYTES, "copy_counter_kib": copy_kib,
                                        "factor": factor}
    for which, rec in out.items():
        t = TRAFFIC[which]
        rec["kernel"] = t["kernel"]
        rec["kernel_source_sha256"] = source_hash(t["src"])
        rec["hbm_bytes_per_launch"] = rec.get("fetch_size_bytes", 0.0) + rec.get("write_size_bytes", 0.0)
        rec["command"] = command
        with open(t["file"], "w") as f:
            json.dump(rec, f, indent=1)
        print("wrote", t["file"], json.dumps({k: rec[k] for k in ("hbm_bytes_per_launch",)}))


def cpu_baseline(x, target_s: float):
    """The fp64 oracle, as it stands, on a bounded row sample of the prefill workload."""
    import numpy as np
    import oracle
    q = oracle._f64(x.q)
    k = oracle._f64(x.k)
    v = oracle._f64(x.v)
    B, Hq, N, d = q.shape

    def sample_flop(step):
        rows = np.arange(0, N, step, dtype=np.float64)
        return 4.0 * d * float((rows + 1).sum()) * B * Hq

    # two short calibration runs (their difference cancels the per-call cost of the
    # oracle's output allocation), then one run sized to about target_s
    times = {}
    for st in (256, 64):
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, True, x.scale, row_step=st)
        times[st] = time.perf_counter() - t0
    dt_cal = times[64] - times[256]
    # a difference within timing noise (under 10 ms) falls back to the larger run's own rate
    rate = ((sample_flop(64) - sample_flop(256)) / dt_cal if dt_cal > 0.01
            else sample_flop(64) / max(times[64], 1e-6))
    step = int(min(256, max(1, round(sample_flop(1) / (rate * target_s)))))
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, True, x.scale, row_step=step)
    dt = time.perf_counter() - t0
    return {"value": sample_flop(step) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads_used(),
            "kind": "oracle",
            "sample": "fp64 plain-definition oracle on %s of all 28 heads of the N=16384 causal "
                      "prefill (%.1f GFLOP, %.1f s wall)" % ("every query row" if step == 1 else "every %dth query row" % step,
                                                             sample_flop(step) / 1e9, dt)}


def host_cpu() -> str:
    """The host's CPU model name, as the kernel reports it (empty if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def host_info() -> dict:
    """What the CPU baseline ran on: the CPU model, the logical CPUs the kernel
    reports (nproc), the ones this process may run on (its affinity mask) and the
    threads the oracle's parallel regions actually use."""
    import oracle
    return {"cpu_model": host_cpu(), "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "oracle_threads": oracle.threads_used()}


def cpu_baseline_decode(dx, nbytes: int):
    """The fp64 oracle, as it stands, on the whole 32k-token decode (one call)."""
    import oracle
    q, kc, vc = oracle._f64(dx.q), oracle._f64(dx.k_cache), oracle._f64(dx.v_cache)
    calls, t0 = 0, time.perf_counter()
    while calls < 3 or time.perf_counter() - t0 < 2.0:  # repeated to about 2 s of wall time
        oracle.decode(q, kc, vc, dx.block_table, dx.seq_lens, dx.scale, dx.page_size, dx.max_blocks)
        calls += 1
    dt = (time.perf_counter() - t0) / calls
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.threads_used(), "kind": "oracle",
            "sample": "fp64 plain-definition oracle on the whole decode (all 28 heads, 32768 cached tokens; "
                      "the cache converted to float64 beforehand), %d calls, %.1f ms each, bytes counted as "
                      "the bf16 cache's" % (calls, dt * 1e3)}


def _timed(fn, min_s: float = 1.0, min_calls: int = 1):
    """Mean wall time of fn() over repeated calls lasting at least min_s."""
    calls, t0 = 0, time.perf_counter()
    while calls < min_calls or time.perf_counter() - t0 < min_s:
        fn()
        calls += 1
    return (time.perf_counter() - t0) / calls, calls


def oracle_table(configs, budget_s: float, threads: int = 0):
    """The fp64 oracle, as it stands, timed on each workload with the inputs already
    converted to float64 (generation and conversion excluded).  Prefill workloads whose
    full run would exceed the budget are timed on every k-th query row of all heads, and
    the full-run time is scaled from that sample by the algorithmic work (the oracle's
    cost per row grows with the row's visible keys, as the work does)."""
    import numpy as np
    import oracle
    from exact_io_aware_prefill_amd import workloads as W

    if threads > 0:
        oracle.set_num_threads(threads)
    rows = {}
    for c in configs:
        t_setup = time.perf_counter()
        if c in ("c1", "c2") or c.startswith("c3-"):
            cfg = W.PREFILL_SMALL_F32 if c == "c1" else W.PREFILL_2K if c == "c2" else W.prefill_long(int(c[3:]))
            x = W.make_prefill(cfg)
            q, k, v = oracle._f64(x.q), oracle._f64(x.k), oracle._f64(x.v)
            B, Hq, N, d = q.shape
            full_flop = 2.0 * B * Hq * d * N * N

            def flop_of(step):
                r = np.arange(0, N, step, dtype=np.float64)
                return 4.0 * d * float((r + 1).sum()) * B * Hq

            step = 1
            if full_flop > 2e10:  # calibrate on a sparse sample, then size the sample to the budget
                probe = max(1, N // 64)
                t0 = time.perf_counter()
                oracle.prefill(q, k, v, True, x.scale, row_step=probe)
                rate = flop_of(probe) / max(time.perf_counter() - t0, 1e-6)
                step = max(1, int(np.ceil(full_flop / (rate * budget_s))))
            dt, calls = _timed(lambda: oracle.prefill(q, k, v, True, x.scale, row_step=step),
                               min_s=0.5 if step == 1 else 0.0)
            full_s = dt * full_flop / flop_of(step) if step > 1 else dt
            rows[c] = {"workload": cfg["name"], "seconds_full": full_s,
                       "value": full_flop / full_s / 1e12, "unit": "TFLOP/s",
                       "sample": "all rows" if step == 1 else "every %dth query row of all %d heads (%.1f s), "
                                 "scaled to the full run by work" % (step, Hq, dt),
                       "calls": calls}
        elif c in ("c4", "c5"):
            dx = W.make_decode_32k() if c == "c4" else W.make_decode_paged()
            qd, kc, vc = oracle._f64(dx.q), oracle._f64(dx.k_cache), oracle._f64(dx.v_cache)
            lens = dx.seq_lens.numpy().astype(np.int64)
            Hkv, d = kc.shape[2], kc.shape[3]
            nbytes = float(lens.sum()) * Hkv * d * 2 * 2  # K and V rows attended, as bf16
            dt, calls = _timed(lambda: oracle.decode(qd, kc, vc, dx.block_table, dx.seq_lens, dx.scale,
                                                     dx.page_size, dx.max_blocks), min_s=1.0)
            rows[c] = {"workload": (W.DECODE_32K if c == "c4" else W.DECODE_PAGED)["name"], "seconds_full": dt,
                       "value": nbytes / dt / 1e9, "unit": "GB/s (bf16 K/V bytes attended)", "sample": "whole call",
                       "calls": calls}
        else:
            raise SystemExit("unknown workload %r" % c)
        rows[c]["elapsed_s"] = round(time.perf_counter() - t_setup, 1)  # generation, conversion and timing
        print("oracle %s: %s" % (c, json.dumps(rows[c])), file=sys.stderr, flush=True)
    return {"threads": oracle.threads_used(), "host": host_info(), "workloads": rows}


def settle(fn, ms: float) -> None:
    """Untimed launches of `fn` for about `ms` milliseconds (one timed launch sets the
    count).  From a cold start the shader clock under the prefill climbs over the
    first few dozen launches (16k prompt: 951 TFLOP/s over launches 0-4, 1201 over
    5-24, 1219-1227 from 25 to 400, 1211-1213 after a second), so a leg timed right
    away would measure the climb rather than the clock a sustained run holds."""
    import torch
    if ms <= 0:
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(int(ms / max(e0.elapsed_time(e1), 1e-3))):
        fn()
    torch.cuda.synchronize()


def prefill_sweep(attn, W, dev, steps: int, warmup: int) -> dict:
    """The causal prefill alone at the prompt lengths of the short-prompt workload
    (N = 2048) and the long-prompt sweep (8192, 16384, 30720).  Each length first runs
    untimed launches for at least 0.3 s (and `warmup` of them), so the shader clock has
    settled under this load, then at least `steps` launches and 0.3 s between two
    events.  Which instantiation runs follows from the launch size: the key split at
    N = 2048 (448 workgroups), the plain kernel above."""
    import torch
    out = {"metric": "causal prefill TFLOP/s by prompt length", "unit": "TFLOP/s", "steps": steps,
           "warmup": warmup, "data": "synthetic", "results": []}
    for cfg in (W.PREFILL_2K, W.prefill_long(8192), W.prefill_long(16384), W.prefill_long(30720)):
        px = W.make_prefill(cfg)
        q, k, v = (t.to(dev) for t in (px.q, px.k, px.v))
        B, Hq, N, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        def run(n: int) -> float:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                attn.attn_prefill(q, k, v, o, lse, True, px.scale)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        first = run(1)
        run(max(warmup, int(300.0 / first) + 1))
        n = max(steps, int(300.0 / first) + 1)
        ms = run(n)
        flop = 2.0 * B * Hq * d * N * N
        out["results"].append({"workload": cfg["name"], "N": N, "launches": n, "ms_per_launch": ms,
                               "value": flop / (ms * 1e-3) / 1e12,
                               "frac": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
        del q, k, v, o, lse, px
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.oracle_table:
        print(json.dumps(oracle_table(args.oracle_configs.split(","), args.oracle_budget, args.oracle_threads)), flush=True)
        return
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.traffic_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path here runs on a single MI355X "
              "and has no multi-GPU mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_io_aware_prefill_amd import attn
    from exact_io_aware_prefill_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.prefill_sweep:
        print(json.dumps(prefill_sweep(attn, W, dev, args.steps, args.warmup)), flush=True)
        return

    pcfg = W.prefill_long(16384)
    px = W.make_prefill(pcfg)
    q, k, v = (t.to(dev) for t in (px.q, px.k, px.v))
    B, Hq, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    prefill_flop = 2.0 * B * Hq * d * N * N

    dcfg = W.DECODE_32K
    dx = W.make_decode_32k(dcfg)
    dq = dx.q.to(dev)
    kc0, vc0 = dx.k_cache.to(dev), dx.v_cache.to(dev)
    kcs = [kc0] + [kc0.clone() for _ in range(N_KV_COPIES - 1)]  # distinct allocations
    vcs = [vc0] + [vc0.clone() for _ in range(N_KV_COPIES - 1)]
    sl = dx.seq_lens.to(dev)
    do = torch.empty_like(dq)
    dl = torch.empty((dq.shape[0], dq.shape[1]), dtype=torch.float32, device=dev)
    chunk = dcfg["chunk"]
    wsb = attn.attn_decode_workspace_bytes(dq.shape[0], dq.shape[1], kcs[0].shape[2], d, dx.page_size,
                                           dx.max_blocks, chunk)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    decode_bytes = (kcs[0].numel() + vcs[0].numel()) * 2 + dq.numel() * 2 + do.numel() * 2 + dl.numel() * 4

    def run_prefill():
        attn.attn_prefill(q, k, v, o, lse, True, px.scale)

    def run_decode(i):
        attn.attn_decode(dq, kcs[i % N_KV_COPIES], vcs[i % N_KV_COPIES], None, sl, do, dl, dx.page_size,
                         dx.max_blocks, dx.scale, chunk, ws)

    do_p = args.only in (None, "prefill")
    do_d = args.only in (None, "decode")
    # FP8 prefill of the same prompt (E4M3 inputs), timed on its own before the step
    # loop.  Each prefill leg first runs its own kernel untimed for --settle-ms, so
    # its W warm-up and K timed launches see the clock a sustained run holds
    fp8 = None
    if args.only in (None, "fp8") and not args.no_fp8:
        fx = W.prefill_fp8_inputs(pcfg["seed"], B, Hq, k.shape[1], N, d)
        q8, k8, v8 = fx.q8.to(dev), fx.k8.to(dev), fx.v8.to(dev)
        dsq, dsk, dsv = fx.descale_q.to(dev), fx.descale_k.to(dev), fx.descale_v.to(dev)
        o8 = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
        l8 = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)

        def run_fp8():
            attn.attn_prefill_fp8(q8, k8, v8, o8, l8, dsq, dsk, dsv, True, fx.scale)
        settle(run_fp8, args.settle_ms)
        for _ in range(args.warmup):
            run_fp8()
        torch.cuda.synchronize()
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev8[i][0].record()
            run_fp8()
            ev8[i][1].record()
        torch.cuda.synchronize()
        fp8_ms = sum(e[0].elapsed_time(e[1]) for e in ev8) / args.steps
        a8 = prefill_flop / (fp8_ms * 1e-3) / 1e12
        fp8 = {"value": a8, "unit": "TFLOP/s", "avg_launch_ms": fp8_ms, "dtype": "fp8-e4m3 in, bf16 out",
               "config": {"workload": pcfg["name"].replace("bf16", "fp8e4m3"), "descales": "per (sequence, KV head)"},
               "roofline": {"bound": "mfma", "achieved": a8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                            "frac": a8 / PEAK_FP8_TFLOPS, "traffic": measured_traffic("fp8"),
                            "kernel": "prefill_fp8_kernel<128, false, false>", "algorithmic_flop_per_launch": prefill_flop}}

    if do_p:
        settle(run_prefill, args.settle_ms)
    for i in range(args.warmup):
        if do_p:
            run_prefill()
        if do_d:
            run_decode(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        if do_p:
            run_prefill()
        evs[i][1].record()
        if do_d:
            run_decode(i)
        evs[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    # Decode throughput: back-to-back calls (rotating the KV copies) inside one pair
    # of events on the launch stream.  The per-step events above put an event
    # between every two calls, which adds a few microseconds to a ~20 us call.
    dec_bb_ms = None
    if do_d:
        reps = 5 * args.steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            run_decode(i)
        e1.record()
        torch.cuda.synchronize()
        dec_bb_ms = e0.elapsed_time(e1) / reps

    # Floor of the decode call, timed the same way (back-to-back, rotating the same KV
    # copies): one kernel that reads the K and V caches once on the split kernel's
    # grid (one 256-thread workgroup per (chunk, KV head)), then the same read followed
    # by an empty dependent launch, the least a two-kernel split + combine can cost.
    floor = None
    if do_d:
        wgs = -(-kcs[0].shape[1] // chunk) * kcs[0].shape[2]
        sink = torch.zeros(4 * wgs, dtype=torch.int32, device=dev)
        reps = 5 * args.steps

        def time_calls(fn):
            for i in range(10):
                fn(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        def read(i):
            attn.attn_bench_stream_read(kcs[i % N_KV_COPIES], vcs[i % N_KV_COPIES], wgs, sink)

        def read_and_launch(i):
            read(i)
            attn.attn_bench_empty()
        read_ms = time_calls(read)
        read2_ms = time_calls(read_and_launch)
        # the same read on other grids: the fastest plain read of these bytes here
        sweep = {}
        for g in READ_GRIDS:
            gsink = torch.zeros(4 * g, dtype=torch.int32, device=dev)
            sweep[g] = time_calls(lambda i, g=g, gsink=gsink: attn.attn_bench_stream_read(
                kcs[i % N_KV_COPIES], vcs[i % N_KV_COPIES], g, gsink))
        gbest = min(sweep, key=sweep.get)
        floor = {"read_ms": read_ms, "read_GBps": decode_bytes / (read_ms * 1e-3) / 1e9,
                 "read_plus_launch_ms": read2_ms, "workgroups": wgs,
                 "best_read": {"ms": sweep[gbest], "GBps": decode_bytes / (sweep[gbest] * 1e-3) / 1e9,
                               "workgroups": gbest, "grids_tried": list(READ_GRIDS)},
                 "what": "one kernel reading the decode's K and V caches once (16-byte loads, grid-stride, %d "
                         "workgroups of 256 threads, the split kernel's grid), then the same read followed by an "
                         "empty dependent launch; %d back-to-back calls between two events, rotating the %d KV copies"
                         % (wgs, reps, N_KV_COPIES)}

    # Decode over an E4M3 copy of the same 32k cache (one byte per element), timed as
    # the bf16 decode: back-to-back calls rotating the copies, between two events
    fp8_dec = None
    if do_d and not args.no_fp8:
        fd = W.decode_fp8_inputs(dcfg["seed"], 1, dq.shape[1], kcs[0].shape[2], d, [kcs[0].shape[1]],
                                 kcs[0].shape[1], False)
        k8s = [fd.k_cache8.to(dev)] + [None] * (N_KV_COPIES - 1)
        v8s = [fd.v_cache8.to(dev)] + [None] * (N_KV_COPIES - 1)
        for i in range(1, N_KV_COPIES):
            k8s[i], v8s[i] = k8s[0].clone(), v8s[0].clone()
        q8d, dsk, dsv = fd.q.to(dev), fd.descale_k.to(dev), fd.descale_v.to(dev)
        o8d = torch.empty_like(q8d)
        l8d = torch.empty((q8d.shape[0], q8d.shape[1]), dtype=torch.float32, device=dev)

        def run_decode8(i):
            attn.attn_decode_fp8(q8d, k8s[i % N_KV_COPIES], v8s[i % N_KV_COPIES], dsk, dsv, None, sl, o8d, l8d,
                                 fd.page_size, fd.max_blocks, fd.scale, chunk, ws)
        for i in range(args.warmup):
            run_decode8(i)
        reps = 5 * args.steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            run_decode8(i)
        e1.record()
        torch.cuda.synchronize()
        ms8 = e0.elapsed_time(e1) / reps
        bytes8 = (k8s[0].numel() + v8s[0].numel()) + q8d.numel() * 2 + o8d.numel() * 2 + l8d.numel() * 4
        fp8_dec = {"value": bytes8 / (ms8 * 1e-3) / 1e9, "unit": "GB/s", "avg_ms": ms8,
                   "timing": "%d back-to-back calls between two events" % reps,
                   "dtype": "fp8-e4m3 cache, bf16 q/o",
                   "roofline": {"bound": "hbm", "achieved": bytes8 / (ms8 * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": bytes8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "kernels": "decode_split_kernel<128, false, false, true, false> + lse_combine_kernel<128, false, 2>",
                                "algorithmic_bytes_per_launch": bytes8},
                   "speedup_vs_bf16_cache": dec_bb_ms / ms8}

    # Batched paged decode: 32 sequences with lengths uniform in [1024, 32768], 32/8
    # heads, 16-token pages placed by a seeded permutation of one shared pool.  The
    # lengths and block table are the paged workload's own (its seeded draws); the K/V
    # values are drawn on the device (N(0,1), bf16), which keeps the leg short.  The
    # pool (about 2.2 GB) is far larger than the Infinity Cache, so no copies are
    # rotated.  Timed as the 32k decode (back-to-back calls between two events), with
    # its own floor: the same read kernel over the whole pool on the split kernel's grid.
    paged = None
    if do_d and not args.no_paged:
        pc = W.DECODE_PAGED
        pq, pbt, psl, pool, pmb = W.decode_paged_layout(pc["seed"], pc["B"], pc["Hq"], pc["d"], pc["page_size"],
                                                         pc["len_min"], pc["len_max"])
        gen = torch.Generator(device=dev)
        gen.manual_seed(pc["seed"])
        pshape = (pool, pc["page_size"], pc["Hkv"], pc["d"])
        pk = torch.randn(pshape, generator=gen, device=dev, dtype=torch.bfloat16)
        pv = torch.randn(pshape, generator=gen, device=dev, dtype=torch.bfloat16)
        pqd, pbtd, psld = pq.to(dev), pbt.to(dev), psl.to(dev)
        pod = torch.empty_like(pqd)
        pld = torch.empty((pc["B"], pc["Hq"]), dtype=torch.float32, device=dev)
        pchunk = 0  # automatic: the balanced split, for a batch
        pws = torch.empty(attn.attn_decode_workspace_bytes(pc["B"], pc["Hq"], pc["Hkv"], pc["d"], pc["page_size"],
                                                           pmb, pchunk), dtype=torch.uint8, device=dev)
        pscale = 1.0 / math.sqrt(pc["d"])

        def run_paged():
            attn.attn_decode(pqd, pk, pv, pbtd, psld, pod, pld, pc["page_size"], pmb, pscale, pchunk, pws)

        def time_back_to_back(fn, reps):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        preps = max(10, args.steps)
        pms = time_back_to_back(run_paged, preps)
        pbytes = (int(psl.to(torch.int64).sum()) * pc["Hkv"] * pc["d"] * 2 * 2 + pqd.numel() * 2 * 2
                  + pld.numel() * 4)
        pgrid = pc["Hkv"] * max(1, BALANCED_WORKGROUPS // pc["Hkv"])  # the balanced split's grid
        psink = torch.zeros(4 * pgrid, dtype=torch.int32, device=dev)
        pool_bytes = pk.numel() * 2
        pread_ms = time_back_to_back(lambda: attn.attn_bench_stream_read(pk, pv, pgrid, psink), preps)
        psweep = {}
        for g in READ_GRIDS:
            gsink = torch.zeros(4 * g, dtype=torch.int32, device=dev)
            psweep[g] = time_back_to_back(lambda g=g, gsink=gsink: attn.attn_bench_stream_read(pk, pv, g, gsink),
                                          preps)
        pbest = min(psweep, key=psweep.get)
        pgbs = pbytes / (pms * 1e-3) / 1e9
        paged = {"value": pgbs, "unit": "GB/s", "avg_ms": pms,
                 "timing": "%d back-to-back calls between two events" % preps,
                 "config": {"workload": pc["name"], "batch": pc["B"], "q_heads": pc["Hq"], "kv_heads": pc["Hkv"],
                            "head_dim": pc["d"], "page_size": pc["page_size"],
                            "cached_tokens": int(psl.to(torch.int64).sum()),
                            "split": "balanced (equal shares of each KV head's tokens, %d workgroups)" % pgrid,
                            "values": "lengths and block table of the paged workload; K/V drawn on the device"},
                 "roofline": {"bound": "hbm", "achieved": pgbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": pgbs / PEAK_HBM_GBS, "traffic": measured_traffic("paged"),
                              "kernels": "decode_split_kernel<128, false, false, false, true> + lse_combine_kernel<128, true, 1>",
                              "algorithmic_bytes_per_launch": pbytes},
                 "floor": {"read_ms": pread_ms, "read_GBps": 2 * pool_bytes / (pread_ms * 1e-3) / 1e9,
                           "workgroups": pgrid,
                           "what": "one kernel reading the whole K and V page pools once (%d bytes; 16-byte loads, "
                                   "grid-stride, %d workgroups of 256 threads, the split kernel's count), %d "
                                   "back-to-back calls between two events" % (2 * pool_bytes, pgrid, preps),
                           "call_over_read": pms / pread_ms,
                           "best_read": {"ms": psweep[pbest], "GBps": 2 * pool_bytes / (psweep[pbest] * 1e-3) / 1e9,
                                         "workgroups": pbest, "grids_tried": list(READ_GRIDS)}}}
        del pk, pv

    if args.copy_calibration:  # reference dispatch for the HBM byte counters: copy 1 GiB
        src = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": (prefill_flop / (pre_ms * 1e-3) / 1e12) if do_p else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pcfg["name"] + " + " + dcfg["name"],
                   "prefill": {"batch": B, "q_heads": Hq, "kv_heads": k.shape[1], "seq_len": N,
                               "head_dim": d, "causal": True},
                   "decode": {"batch": 1, "q_heads": dq.shape[1], "kv_heads": kcs[0].shape[2],
                              "cache_tokens": kcs[0].shape[1], "head_dim": d, "chunk_tokens": chunk,
                              "splits": -(-kcs[0].shape[1] // chunk), "kv_copies_rotated": N_KV_COPIES}},
    }
    if do_p:
        achieved = prefill_flop / (pre_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("prefill"),
                           "kernel": "prefill_bf16_kernel<128, false, 1, 3>", "avg_launch_ms": pre_ms,
                           "algorithmic_flop_per_launch": prefill_flop}
    if do_d:
        gbs = decode_bytes / (dec_bb_ms * 1e-3) / 1e9
        out["decode"] = {"value": gbs, "unit": "GB/s", "avg_ms": dec_bb_ms,
                         "timing": "%d back-to-back calls between two events" % (5 * args.steps),
                         "avg_ms_events_around_each_call": dec_ms,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("decode"),
                                      "kernels": "decode_split_kernel<128, false, false, false, false> + lse_combine_kernel<128, false, 2>",
                                      "algorithmic_bytes_per_launch": decode_bytes}}
        if floor is not None:
            floor["call_over_read_plus_launch"] = dec_bb_ms / floor["read_plus_launch_ms"]
            out["decode"]["floor"] = floor
    if fp8 is not None:
        out["fp8_prefill"] = fp8
    if fp8_dec is not None:
        out["fp8_decode"] = fp8_dec
    if paged is not None:
        out["decode_paged"] = paged
    if do_p and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(px, args.cpu_seconds)
        out["cpu_baseline"]["host"] = host_info()
    if do_d and not args.no_cpu_baseline:
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(dx, decode_bytes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
