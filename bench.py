#!/usr/bin/env python3
"""Throughput of tiled exact attention, forward + backward, on one MI355X.

One step = the whole path over one batch of the workload: fa_fwd, then the two
backward stages fa_bwd_dq and fa_bwd_dkdv, all through the C ABI (with
--backward single-pass: fa_bwd with FA_BWD_ATOMIC_DQ instead).  Default
workload: GPT-2-medium-shaped attention, B=64 H=16 N=1024 d=64, fp16, causal,
scale 1/8 (the shape of the paper's headline measurement), synthetic seeded
inputs already resident in HBM.

Reported value: fwd+bwd TFLOP/s with matrix-core FLOPs counted over kept
(query, key) pairs -- 4 d per pair forward and 10 d per pair backward
(Q K^T, P V; the score recompute, dV, dP, dK, dQ).  The backward's extra
score/dP recompute in the dQ kernel is work done but not credited.

Before the warm-up steps the step runs untimed for --settle-ms (300 ms by
default) so that the timed region sees the GPU's sustained clocks rather than
their ramp; the JSON line reports the value it used.

Prints ONE JSON line (plus a few human-readable lines on stderr).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (B64·H16·N1024·d64 fp16 causal), % of MFMA peak"
DEFAULT_WORKLOAD = "gpt2_medium"  # the configuration METRIC is quoted on
# MI355X published peaks: dense fp16/bf16 matrix 2.5 PFLOP/s (= 256 CUs x 4096
# FLOP/clk x 2.4 GHz), HBM3E 8 TB/s.
PEAK_MFMA_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 2 * PEAK_MFMA_TFLOPS  # dense E4M3 matrix rate, twice the 16-bit one


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
DROPOUT_SEED = 2024  # generator seed of the dropout workload's keep mask
KERNEL_SOURCES = os.path.join(ROOT, "io_aware_exact_fwd_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the forward, dQ and dK/dV kernels are compiled from (their
# translation units and every header those include)
TRAFFIC_SOURCES = ("fa_bwd.hip", "fa_common.hpp", "fa_dropout.hpp", "fa_fwd.hip", "fa_kernels.hpp",
                   "fa_tiles.hpp")


def source_digest():
    """sha256 over the sources of the kernels whose HBM traffic is recorded;
    measured traffic is only reported while it matches the digest recorded
    with the counters."""
    import hashlib

    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(KERNEL_SOURCES, name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("source_sha256") != source_digest():
        return None
    k = rec.get("kernels", {}).get(f"{kernel}/{workload}")
    return None if k is None else k.get("bytes_per_launch")


def kernel_work(w):
    """Per-launch algorithmic work of each kernel of the step (FLOPs, bytes).

    Units: kept (query, key) pairs.  fwd: Q K^T and P V = 4 d FLOP/pair.
    dq kernel: S, dP and dQ products = 6 d FLOP/pair.  dkdv kernel: S, dP, dV,
    dK products = 8 d FLOP/pair.  Bytes: each tensor the kernel must read or
    write, once."""
    from io_aware_exact_fwd_amd.workloads import kept_pairs_per_head

    pairs = kept_pairs_per_head(w.N, w.causal, w.block_mask(), w.mask_block, w.window) * w.B * w.H
    x = w.B * w.H * w.N * w.d * w.elem_bytes      # one (B, H, N, d) tensor
    xkv = w.B * w.H_kv * w.N * w.d * w.elem_bytes  # one K/V-shaped tensor
    n4 = w.B * w.H * w.N * 4                      # one float32 (B, H, N) vector
    return {
        "fwd": {"flops": 4.0 * w.d * pairs, "bytes": 2 * x + 2 * xkv + n4},       # Q K V -> O, LSE
        "dq": {"flops": 6.0 * w.d * pairs, "bytes": 4 * x + 2 * xkv + 2 * n4},    # Q K V O dO LSE -> dQ D
        "dkdv": {"flops": 8.0 * w.d * pairs, "bytes": 2 * x + 4 * xkv + 2 * n4},  # Q K V dO LSE D -> dK dV
        # single-pass backward (pre-pass, dK/dV with atomic dQ, conversion): S, dP,
        # dV, dK, dQ products = 10 d FLOP/pair; Q K V O dO LSE -> dQ dK dV
        "bwd": {"flops": 10.0 * w.d * pairs, "bytes": 4 * x + 4 * xkv + n4},
    }


class ClockSampler:
    """Samples the GPU shader clock (the current level of the kernel's
    pp_dpm_sclk table, marked '*') every few milliseconds on a host thread
    while the timed steps run; mean() is None where the file is absent."""

    def __init__(self, period_s=0.004):
        import glob
        import threading

        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if files else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            try:
                with open(self.path) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            mhz = float(line.split(":")[1].strip().split("Mhz")[0])
                            if mhz > 400:  # skip the idle / deep-sleep level
                                self.samples.append(mhz)
            except (OSError, ValueError, IndexError):
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def mean(self):
        return round(sum(self.samples) / len(self.samples), 1) if self.samples else None


def settle(step, ms):
    """Run `step` untimed for at least `ms` milliseconds of wall time before
    the warm-up steps: the GPU raises its clocks over the first tens of
    milliseconds of sustained load, and a short timed region would otherwise
    measure that ramp rather than the steady rate."""
    import torch

    if ms <= 0:
        return 0
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        step()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def decode_bench(w, args, dev):
    """Decode workload: n_q queries per head against N keys.  Bound by HBM:
    its algorithmic bytes are K and V once plus Q, O and LSE.  Prints one
    JSON line like the headline path."""
    import torch

    from io_aware_exact_fwd_amd import fa_fwd_decode
    from io_aware_exact_fwd_amd.workloads import make_decode_inputs

    q, k, v = (t.to(dev) for t in make_decode_inputs(w.B, w.H, w.N, w.d, w.nq, w.dtype,
                                                      hkv=w.H_kv))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.nq), dtype=torch.float32, device=dev)
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} H_kv={w.H_kv} N={w.N} n_q={w.nq} d={w.d} "
        f"{w.dtype} causal={w.causal}; warmup {args.warmup}, steps {args.steps}")
    settle(lambda: fa_fwd_decode(q, k, v, causal=w.causal, scale=w.scale, window=w.window,
                                 out=o, lse=lse), args.settle_ms)
    for _ in range(args.warmup):
        fa_fwd_decode(q, k, v, causal=w.causal, scale=w.scale, window=w.window, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        fa_fwd_decode(q, k, v, causal=w.causal, scale=w.scale, window=w.window, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    e = 2  # bf16 / fp16
    nbytes = 2 * w.B * w.H_kv * w.N * w.d * e + 2 * w.B * w.H * w.nq * w.d * e + w.B * w.H * w.nq * 4
    gbs = nbytes / (ms_step / 1e3) / 1e9
    log(f"[bench] decode {ms_step * 1e3:.1f} us per call ({ms_ev * 1e3:.1f} us by events), "
        f"{nbytes / 1e6:.1f} MB -> {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM peak)")
    out = {
        "metric": f"decode attention forward HBM GB/s ({w.name})", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "n_q": w.nq,
                   "d": w.d, "dtype": w.dtype, "causal": w.causal, "scale": w.scale},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": round(ms_ev and nbytes / (ms_ev / 1e3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (ms_ev / 1e3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def fp8_bench(w, args, dev):
    """FP8 workload: one step = quantise Q, K, V (rotation + block scales)
    then attention on the codes.  value = forward FLOPs of the attention /
    step time; the attention kernel is rated against the dense FP8 matrix
    peak, the quantiser against HBM (bf16 in, one byte per element out)."""
    import torch

    from io_aware_exact_fwd_amd import fa_fwd_fp8, fp8_quantize
    from io_aware_exact_fwd_amd.binding import lib, _stream
    from io_aware_exact_fwd_amd.workloads import fwd_flops, make_inputs, make_signs

    q, k, v, _ = (t.to(dev) for t in make_inputs(w.B, w.H, w.N, w.d, w.dtype, hkv=w.H_kv))
    signs = make_signs(w.d).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    p, ws = fp8_quantize(q, k, v, signs, w.causal, w.scale, w.window)
    L = lib()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        st = L.fa_fp8_quantize(ctypes.byref(p), signs.data_ptr(), q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q))
        if ev is not None:
            ev[1].record()
        st |= L.fa_fwd_fp8(ctypes.byref(p), signs.data_ptr(), ws.data_ptr(), ws.numel(),
                           o.data_ptr(), lse.data_ptr(), _stream(q))
        if ev is not None:
            ev[2].record()
        if st:
            raise RuntimeError(f"FP8 path failed ({st})")

    log(f"[bench] workload {w.name}: B={w.B} H={w.H} H_kv={w.H_kv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal}, FP8 path; warmup {args.warmup}, steps {args.steps}")
    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_q = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms_a = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    ms_step = wall * 1e3 / args.steps
    flops = fwd_flops(w)
    value = flops / (ms_step / 1e3) / 1e12
    elems = (w.B * w.H + 2 * w.B * w.H_kv) * w.N * w.d
    qbytes = elems * (2 + 1)
    ach = flops / (ms_a / 1e3) / 1e12
    log(f"[bench] quantise {ms_q * 1e3:.1f} us ({qbytes / (ms_q / 1e3) / 1e9:.0f} GB/s), "
        f"attention {ms_a * 1e3:.1f} us ({ach:.1f} TFLOP/s, {100 * ach / PEAK_FP8_TFLOPS:.1f}% "
        f"of the FP8 peak); step {ms_step * 1e3:.1f} us -> {value:.1f} TFLOP/s")
    out = {
        "metric": f"FP8 attention forward TFLOP/s ({w.name})", "value": round(value, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "d": w.d,
                   "dtype": w.dtype, "causal": w.causal, "scale": w.scale},
        "kernel_ms": {"fp8_quantize": round(ms_q, 5), "fp8_fwd": round(ms_a, 5)},
        "sclk_mhz": clock.mean(),
        "roofline": {"kernel": "fp8_fwd", "bound": "mfma", "achieved": round(ach, 1),
                     "peak": round(PEAK_FP8_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def roofline(name, work, ms):
    """Roofline entry for one kernel: bound = the larger of its compulsory-byte
    time at peak HBM and its FLOP time at peak matrix rate."""
    t_hbm = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = work["flops"] / (PEAK_MFMA_TFLOPS * 1e12)
    sec = ms / 1e3
    if t_hbm > t_mfma:
        ach = work["bytes"] / sec / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    ach = work["flops"] / sec / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1),
            "peak": round(PEAK_MFMA_TFLOPS, 1), "unit": "TFLOP/s",
            "frac": round(ach / PEAK_MFMA_TFLOPS, 4), "traffic": None}


def cpu_baseline(w, inputs, seconds):
    """Time the fp64 oracle (as it stands) on whole heads of the same workload
    until `seconds` have passed; report its fwd+bwd rate in the metric's unit."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from io_aware_exact_fwd_amd.workloads import kept_pairs_per_head
    from oracle import attention_backward, attention_forward

    q, k, v, do = inputs
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    bm = w.block_mask()
    grp = w.H // w.H_kv
    ext = dict(window=w.window)
    if w.dropout:
        ext.update(dropout_p=w.dropout, seed=DROPOUT_SEED, offset=0)
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        qn, don = (t[b, h].float().numpy() for t in (q, do))
        kn, vn = (t[b, h // grp].float().numpy() for t in (k, v))
        attention_forward(qn, kn, vn, w.scale, w.causal, bm, w.mask_block, **ext)
        attention_backward(qn, kn, vn, don, w.scale, w.causal, bm, w.mask_block, **ext)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    flops = 14.0 * w.d * kept_pairs_per_head(w.N, w.causal, bm, w.mask_block, w.window) * done
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of {w.name}, fwd+bwd, numpy float64, "
                      f"{el:.1f} s on {len(os.sched_getaffinity(0))} host cores "
                      f"({platform.processor() or platform.machine()})"}


def _short(name):
    for key in ("f32_", "fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_prep_kernel",
                "dq_convert_kernel", "mask_compile"):
        if key in name:
            return key + name[name.find(key) + len(key):][:40]
    return name[:60]


def summarize_stats(path):
    import csv

    rows = list(csv.DictReader(open(path)))
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        print(f"{_short(r['Name']):60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
              f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
              f"{float(r['Percentage']):6.2f}")


def summarize_pmc(path):
    import collections
    import csv

    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        k = _short(r["Kernel_Name"])
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    for k in agg:
        n = len(disp[k])
        vals = " ".join(f"{c}={v / n:.6g}" for c, v in sorted(agg[k].items()))
        print(f"{k:60s} dispatches={n} per-dispatch: {vals}")


def _counter_means(path, counter):
    """Per-kernel mean of one counter (KiB per dispatch) from a rocprofv3
    counter_collection.csv."""
    import collections
    import csv

    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        tot[r["Kernel_Name"]] += float(r["Counter_Value"])
        disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def record_traffic(fetch_csv, write_csv, cfetch_csv, cwrite_csv, workload):
    """Calibrate FETCH_SIZE / WRITE_SIZE against the copy probe (512 MiB read
    and written per launch), scale the attention kernels' counters to HBM
    bytes per launch, write profiles/traffic.json with the digest of the
    kernel sources, and print a summary."""
    copy_kib = 512 * 1024
    cf = [v for k, v in _counter_means(cfetch_csv, "FETCH_SIZE").items() if "elementwise" in k]
    cw = [v for k, v in _counter_means(cwrite_csv, "WRITE_SIZE").items() if "elementwise" in k]
    if not cf or not cw:
        raise SystemExit("copy-probe counters not found")
    fs, ws = copy_kib / max(cf), copy_kib / max(cw)
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    from io_aware_exact_fwd_amd.workloads import WORKLOADS

    work = kernel_work(WORKLOADS[workload])
    rec = {"source_sha256": source_digest(), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "calibration": f"plain elementwise copy (torch.mul(x, 1.0, out=y)) of 512 MiB fp16: "
                          f"FETCH_SIZE {max(cf):.0f} KiB per launch for {copy_kib} KiB read, "
                          f"WRITE_SIZE {max(cw):.0f} KiB for {copy_kib} KiB written",
           "kernels": {}}
    print(f"# calibration: fetch scale {fs:.4f}, write scale {ws:.4f}")
    for key, tag in (("fwd", "fwd_kernel"), ("dq", "bwd_dq_kernel"), ("dkdv", "bwd_dkdv_kernel")):
        fk = [v for k, v in fetch.items() if tag in k and "f32" not in k]
        wk = [v for k, v in write.items() if tag in k and "f32" not in k]
        if not fk or not wk:
            continue
        b = int(round((fs * fk[0] + ws * wk[0]) * 1024))
        rec["kernels"][f"{key}/{workload}"] = {"fetch_kib_raw": round(fk[0]), "write_kib_raw": round(wk[0]),
                                              "bytes_per_launch": b}
        print(f"#   {key:5s} FETCH {fk[0]:10.0f} KiB  WRITE {wk[0]:10.0f} KiB  -> {b / 1e6:8.1f} MB per launch "
              f"(compulsory {work[key]['bytes'] / 1e6:.1f} MB)")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"# wrote {os.path.relpath(TRAFFIC_FILE, ROOT)}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed run of the step before the warm-up steps, in ms of wall "
                         "time (clock ramp-up; 0 to skip)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--backward", choices=("two-kernel", "single-pass"), default="two-kernel",
                    help="backward design: the dQ and dK/dV kernels (default), or one key-outer "
                         "pass with dQ summed by float32 atomics (FA_BWD_ATOMIC_DQ)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU budget of the oracle baseline (0 to skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain elementwise copy of 2 x 512 MiB (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="print a summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--summarize-pmc", metavar="CSV",
                    help="print per-kernel means of a rocprofv3 counter_collection.csv and exit")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn four counter_collection.csv files (FETCH_SIZE and WRITE_SIZE of "
                         "the bench, then of --copy-probe) into profiles/traffic.json and exit")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(*args.record_traffic, args.workload)
        return

    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention shards over (batch, head) with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from io_aware_exact_fwd_amd import bwd_workspace, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_into, fa_fwd
    from io_aware_exact_fwd_amd.workloads import WORKLOADS, bwd_flops, fwd_flops, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        n = 256 * 1024 * 1024  # 512 MiB of fp16 read, 512 MiB written per launch
        x = torch.ones(n, dtype=torch.float16, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 5 launches, each reads {2 * n} B and writes {2 * n} B")
        return
    w = WORKLOADS[args.workload]
    if w.nq:
        decode_bench(w, args, dev)
        return
    if w.fp8:
        fp8_bench(w, args, dev)
        return
    inputs = make_inputs(w.B, w.H, w.N, w.d, w.dtype, hkv=w.H_kv)
    q, k, v, do = (t.to(dev) for t in inputs)
    bm = w.block_mask()
    bmd = None if bm is None else torch.as_tensor(bm, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # the workload's window, grouped K/V heads (through k's shape) and dropout
    ext = dict(window=w.window)
    if w.dropout:
        ext.update(dropout_p=w.dropout, seed=DROPOUT_SEED, offset=0)
    # one workspace for the whole step: the forward compiles the block lists
    # into it and the backward reuses them (FA_REUSE_LISTS)
    single = args.backward == "single-pass"
    p, ws, ws_n, bmt = bwd_workspace(q, w.causal, w.scale, bmd, w.mask_block, k=k,
                                     reuse_lists=bmd is not None, atomic_dq=single, **ext)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa_fwd(q, k, v, w.causal, w.scale, bmt, w.mask_block, out=o, lse=lse, workspace=ws, **ext)
        if ev is not None:
            ev[1].record()
        if single:
            fa_bwd_into(p, q, k, v, o, do, lse, dq, dk, dv, ws, ws_n)
        else:
            fa_bwd_dq(p, q, k, v, o, do, lse, dq, ws, ws_n)
        if ev is not None:
            ev[2].record()
        if not single:
            fa_bwd_dkdv(p, q, k, v, do, lse, dk, dv, ws, ws_n)
        if ev is not None:
            ev[3].record()

    log(f"[bench] workload {w.name}: B={w.B} H={w.H} H_kv={w.H_kv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} mask={w.mask} window={w.window} dropout={w.dropout}; "
        f"{args.backward} backward; warmup {args.warmup}, steps {args.steps}")
    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    sclk = clock.mean()

    per = {"fwd": [], "bwd": []} if single else {"fwd": [], "dq": [], "dkdv": []}
    for ev in events:
        per["fwd"].append(ev[0].elapsed_time(ev[1]))
        if single:
            per["bwd"].append(ev[1].elapsed_time(ev[3]))
        else:
            per["dq"].append(ev[1].elapsed_time(ev[2]))
            per["dkdv"].append(ev[2].elapsed_time(ev[3]))
    ms = {kk: sum(vv) / args.steps for kk, vv in per.items()}
    med = {kk: sorted(vv)[len(vv) // 2] for kk, vv in per.items()}

    # one cold step (outside the timed region): a 512 MiB write first evicts
    # the inputs from L2 and the last-level cache
    flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    cold = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    step(cold)
    torch.cuda.synchronize()
    cold_ms = cold[0].elapsed_time(cold[3])
    del flush
    ms_step = wall * 1e3 / args.steps
    f_fwd, f_bwd = fwd_flops(w), bwd_flops(w)
    value = (f_fwd + f_bwd) / (ms_step / 1e3) / 1e12
    work = kernel_work(w)
    dom = max(ms, key=ms.get)
    roof = roofline(dom, work[dom], ms[dom])
    roof["traffic"] = measured_traffic(dom, w.name)

    for kk in ms:
        r = roofline(kk, work[kk], ms[kk])
        log(f"[bench] {kk:5s} {ms[kk] * 1e3:9.1f} us  {r['achieved']:8.1f} {r['unit']} "
            f"({100 * r['frac']:.1f}% of {r['bound']} peak)")
    peak_at_sclk = PEAK_MFMA_TFLOPS * sclk / 2400.0 if sclk else None
    if sclk:
        log(f"[bench] shader clock during the timed steps {sclk:.0f} MHz: peak there "
            f"{peak_at_sclk:.0f} TFLOP/s, {100 * value / peak_at_sclk:.1f}% of it")
    log(f"[bench] step {ms_step * 1e3:.1f} us -> {value:.1f} TFLOP/s "
        f"({100 * value / PEAK_MFMA_TFLOPS:.1f}% of {PEAK_MFMA_TFLOPS:.0f}); fwd alone "
        f"{f_fwd / (ms['fwd'] / 1e3) / 1e12:.1f} TFLOP/s; one cold step (caches flushed) "
        f"{cold_ms * 1e3:.1f} us")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s ...")
        cpu = cpu_baseline(w, inputs, args.cpu_seconds)

    out = {
        "metric": (METRIC if w.name == DEFAULT_WORKLOAD and not single else
                   f"attention fwd+bwd TFLOP/s ({w.name}{', single-pass backward' if single else ''}),"
                   " % of MFMA peak"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "dtype": w.dtype, "causal": w.causal, "scale": w.scale,
                   "block_mask": w.mask,
                   **({"H_kv": w.H_kv} if w.H_kv != w.H else {}),
                   **({"window": w.window} if w.window else {}),
                   **({"dropout": w.dropout} if w.dropout else {}),
                   "backward": args.backward},
        "pct_of_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "sclk_mhz": sclk,
        "pct_of_mfma_peak_at_sclk": round(100 * value / peak_at_sclk, 2) if sclk else None,
        "fwd_tflops": round(f_fwd / (ms["fwd"] / 1e3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / ((ms["bwd"] if single else ms["dq"] + ms["dkdv"]) / 1e3) / 1e12, 2),
        "kernel_ms": {kk: round(vv, 5) for kk, vv in ms.items()},
        "kernel_ms_median": {kk: round(vv, 5) for kk, vv in med.items()},
        "cold_step_ms": round(cold_ms, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
