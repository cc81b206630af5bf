#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step = one moe_layer_forward (router -> top-k -> grouping -> experts ->
combine) over one batch of seeded synthetic input.

Default run: the headline line is c5, the largest single-GPU configuration
(T = 4096 tokens, d = 6144, 256 experts top-8 sigmoid + a Zipf-skewed bias,
F = 2048 + a shared expert, bf16 on the matrix cores); `--steps` / `--warmup`
apply to it.  The c2 decode layer (T = 1, d = 4096, 256 experts, top-6
sqrt(softplus) x1.5, int8 blocks of 32 with an fp16 scale, bf16
activations) is measured after it in the same process, with its own step
count, and carried in the same JSON line under "decode".  `--workload`
measures one workload alone.

Decode steps walk 1024 distinct tokens and rotate over several full copies of
the layer's weights (27 GB for c2), so the 256 MB Infinity Cache cannot serve
one step's expert weights to the next: every step reads its experts from HBM.
Prefill workloads run one layer copy (19 GB, far beyond any cache) on a fixed
batch.

Output: one JSON line.  `value` = tokens per second of the whole timed region
(inputs resident in HBM).  `roofline` describes the dominant kernel (the
gate/up stage): algorithmic bytes (or flops, when the launch's matrix-core
time exceeds its HBM time) per launch divided by its average duration.  The
durations come from HIP events that the library attaches to its own kernel
dispatches on its stream (hipExtLaunchKernel start/stop timestamps, the same
ones a kernel trace reads): during the timed steps for prefill, in a second
eager pass of the same steps for decode, whose ~50 us steps those
per-dispatch timestamps would slow by ~40 us.  `per_step_ms` (p50 / p90) comes
from a third pass with an event between consecutive steps.  `traffic` is the
HBM byte count from rocprofv3 counters recorded in profiles/traffic.json, or
null when that record was taken on a different version of the kernel source.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload,
on all host threads and on one.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0

WORKLOADS = {
    "c2": dict(base="c2", T=1, copies=4, steps=200, warmup=20),
    # c2 with the router look-ahead: consecutive tokens correlated like a
    # layer's input and the next layer's; each step also routes its token with
    # the next step's router and reads the predicted experts' gate/up weights
    # on a second stream, from the end of the step on (same steps also timed
    # without it)
    "c2la": dict(base="c2", T=1, copies=4, steps=200, warmup=20, lookahead=True),
    "c3": dict(base="c3", T=1, copies=4, steps=200, warmup=20),
    "c3t2": dict(base="c3", T=2, copies=4, steps=200, warmup=20),
    "c4": dict(base="c4", T=512, copies=1, steps=20, warmup=5),
    "c5": dict(base="c5", T=4096, copies=1, steps=10, warmup=3),
    # the c2 layer (int8 blocks of 32) with a 512-token prefill batch: the
    # int8 grouped GEMMs
    "c2p": dict(base="c2", T=512, copies=1, steps=10, warmup=3),
    # Compute-bound supplements for the matrix cores: s1 is c5's shared-expert
    # shape alone (one dense SwiGLU over 4096 tokens: one expert, top-1, no
    # shared expert); s2 is c4 with 16384 tokens (about 512 rows per expert).
    "s1": dict(base="c5", T=4096, over=dict(label="s1", E=1, k=1, n_shared=0, bias="none"), copies=1,
               steps=10, warmup=3, bound="mfma"),
    "s2": dict(base="c4", T=16384, over=dict(label="s2"), copies=1, steps=5, warmup=2, bound="mfma"),
}
N_DECODE_TOKENS = 1024
# Row top-k workloads (the indexer's selection; rows x candidates, top-k):
# scores rotate over enough copies that no step finds its row in the 256 MB
# Infinity Cache.
TOPK_WORKLOADS = {
    "i2": dict(copies=8, steps=200, warmup=20),
    "i3": dict(copies=64, steps=400, warmup=40),
}
# The expert GEMMs of c5's hottest experts alone: c5's own routing (the
# library's router on c5's tokens) with every assignment outside the HOT_E
# most-loaded experts dropped, then the grouped gate/up and down over what is
# left (no shared expert).  HOT_E = 10 is 3.9% of the 256 experts, the share the
# skew is calibrated on.
HOT_WORKLOADS = {"c5hot": dict(base="c5", hot=10, steps=20, warmup=5)}


def describe(cfg):
    w = {"q8b32": "int8 blocks of 32 + fp16 scale", "bf16": "bf16", "f32": "fp32"}[cfg["w"]]
    score = "sqrt(softplus) x%.1f" % cfg["scale"] if cfg["score"] == "sqrt_softplus" else "sigmoid"
    if cfg.get("bias", "none") != "none":
        score += "+bias"
    shared = " + shared F=%d" % cfg["Fs"] if cfg["n_shared"] else ", no shared expert"
    return ("%s: T=%d d=%d E=%d top-%d %s F=%d%s, %s weights, %s activations"
            % (cfg["name"], cfg["T"], cfg["d"], cfg["E"], cfg["k"], score, cfg["F"], shared, w, cfg["act"]))


class Hip:
    """The few HIP runtime calls bench needs (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def sync_event(self):
        """An event that only orders streams (the work after it reads no data
        that the work before it writes): no timing and no system-scope fence,
        so recording it writes back and invalidates no cache."""
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0x2 | 0x20000000) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def ms_or_none(self, a, b):
        """Elapsed time between two events, or None if either was never recorded."""
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0:
            return out.value
        self.lib.hipGetLastError()  # clear it, so the library's next launch check does not see it
        return None

    def wait(self, stream, e):
        assert self.lib.hipStreamWaitEvent(ctypes.c_void_p(stream), e, 0) == 0

    def sync(self, e):
        assert self.lib.hipEventSynchronize(e) == 0

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def gen_weights_host(cfg):
    from synth import configs
    L = {w: configs.gen_mat(cfg, w) for w in ("gate", "up", "down", "s_gate", "s_up", "s_down")}
    L["w_router"] = configs.gen_router(cfg)
    L["bias"] = configs.gen_bias(cfg)
    return L


def upload_copies(L, n, torch):
    import numpy as np

    def dev(a):
        if a is None:
            return None
        if isinstance(a, tuple):
            return tuple(dev(p) for p in a)
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    first = {k: dev(v) for k, v in L.items()}
    copies = [first]
    for _ in range(n - 1):
        copies.append({k: (None if v is None else tuple(p.clone() for p in v) if isinstance(v, tuple) else v.clone())
                       for k, v in first.items()})
    return copies


def expert_bytes(cfg, n_mats=3):
    per = cfg["F"] * cfg["d"]
    b = {"q8b32": per + per // 16, "bf16": 2 * per, "f32": 4 * per}[cfg["w"]]
    return n_mats * b


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = "sparse_moe_layer_02_amd/csrc/"
DOMINANT = {  # (path, weights) -> dominant (gate/up) kernel and the sources it is built from
    ("decode", "any"): ("gateup_gemv_decode_kernel",
                        [_CSRC + f for f in ("gemv_ffn.hip", "gemv_dev.h", "common.h", "kernels.h")]),
    ("prefill", "bf16"): ("gateup_mfma_kernel", [_CSRC + f for f in ("grouped_gemm.hip", "gemm_dev.h", "common.h")]),
    ("prefill", "bf16", "256"): ("gateup_dma_kernel",
                                 [_CSRC + f for f in ("grouped_gemm_dma.hip", "dma_dev.h", "gemm_dev.h", "common.h")]),
    ("prefill", "q8b32"): ("gateup_mfma_q8_kernel",
                           [_CSRC + f for f in ("grouped_gemm_q8.hip", "gemm_dev.h", "common.h")]),
    ("prefill", "q8b32", "lds"): ("gateup_q8_dma_kernel",
                                  [_CSRC + f for f in ("grouped_gemm_q8_dma.hip", "dma_dev.h", "gemm_dev.h",
                                                       "common.h")]),
    ("prefill", "any"): ("gateup_gemv_kernel", [_CSRC + f for f in ("gemv_ffn.hip", "gemv_dev.h", "common.h")]),
}


def dominant(path_kind, w, rows_per_expert=None):
    """The gate/up kernel a layer launches.  bf16 prefill layers whose experts
    average 96 rows or more run the 256-row-tile kernels (the library's tile
    rule: T * k >= 96 * E); int8 prefill layers run their gate/up on the GEMVs
    below 1.5 rows per expert (2 * T * k < 3 * E), on the LDS-copy int8 GEMM up
    to 28 rows (when K is a multiple of 256, as in every int8 workload here),
    on the register-staged one above."""
    if path_kind == "prefill" and w == "bf16" and rows_per_expert is not None and rows_per_expert >= 96:
        return DOMINANT[("prefill", "bf16", "256")]
    if path_kind == "prefill" and w == "q8b32" and (rows_per_expert is None or rows_per_expert < 1.5):
        return DOMINANT[("prefill", "any")]  # int8 layers with few rows per expert: the GEMVs
    if path_kind == "prefill" and w == "q8b32" and rows_per_expert <= 28:
        return DOMINANT[("prefill", "q8b32", "lds")]
    return DOMINANT.get((path_kind, w)) or DOMINANT[(path_kind, "any")]


def rows_per_expert(cfg):
    return cfg["T"] * cfg["k"] / cfg["E"]


def traffic_record(path_kind, w, workload, rpe=None):
    """HBM bytes per launch of the dominant kernel from profiles/traffic.json,
    if it was measured on the current kernel source."""
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(rec_path):
        return None
    with open(rec_path) as f:
        recs = json.load(f)
    kname, srcs = dominant(path_kind, w, rpe)
    r = recs.get(workload)
    if not r or r.get("kernel") != kname or r.get("source_sha") != source_sha(srcs):
        return None
    return r.get("hbm_bytes_per_launch")


def _counter_rows(path):
    """(dispatch id, kernel name, counter, value) per dispatch from a rocprofv3
    counter_collection.csv."""
    import csv
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return out


def record_traffic(workload, path_kind, w, fetch_csv, write_csv, copy_bytes, rec_path=None, rpe=None):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch of the dominant kernel.  Each counter is
    scaled by the factor that makes it read right on the plain device copy of
    ``copy_bytes`` (read and written once) that the same command ran."""
    if workload in TOPK_WORKLOADS:
        kname, srcs = "topk_rows_kernel", TOPK_SOURCES
    else:
        kname, srcs = dominant(path_kind, w, rpe)
    res = {"kernel": kname, "source_sha": source_sha(srcs), "copy_bytes": copy_bytes}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = [r for r in _counter_rows(path) if r[2] == counter]
        kern = [v for _, n, _, v in rows if ("::" + kname + "<") in n or ("::" + kname + "(") in n]
        # the probe's three copies are the last copy dispatches of the run
        copy = [v for _, n, _, v in sorted(rows) if "copy" in n.lower()][-3:]
        if not kern or len(copy) < 3:
            raise SystemExit("no %s dispatches of %s or of the copy probe in %s" % (counter, kname, path))
        copy_kib = sum(copy) / len(copy)
        factor = copy_bytes / (copy_kib * 1024.0)
        kib = sum(kern) / len(kern)
        res[key + "_kib_per_launch"] = kib
        res[key + "_copy_kib"] = copy_kib
        res[key + "_factor"] = factor
        res[key + "_bytes_per_launch"] = kib * 1024.0 * factor
        res[key + "_launches"] = len(kern)
    res["hbm_bytes_per_launch"] = res["fetch_bytes_per_launch"] + res["write_bytes_per_launch"]
    rec_path = rec_path or os.path.join(ROOT, "profiles", "traffic.json")
    recs = {}
    if os.path.exists(rec_path):
        with open(rec_path) as f:
            recs = json.load(f)
    recs[workload] = res
    with open(rec_path, "w") as f:
        json.dump(recs, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: res}))


def copy_probe(torch, hip, stream, mib):
    """A plain device copy of known size, three times: the counters' calibration
    kernel and the practical HBM ceiling (bytes read + written per second)."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for _ in range(3):
        b.copy_(a)
    hip.record(e1, stream)
    hip.sync(e1)
    ms = hip.ms(e0, e1)
    hip.destroy(e0)
    hip.destroy(e1)
    del a, b
    return round(3 * 2 * n * 4 / (ms * 1e-3) / 1e9, 1)


def bench_topk_rows(args):
    """Row top-k (moe_topk_rows): one step = one call over every row of the
    workload.  value = rows per second; roofline: the kernel's algorithmic
    bytes (scores read once, indices and values written once) over its average
    dispatch time, taken in a second pass with dispatch events."""
    import numpy as np
    import torch
    import sparse_moe_layer_02_amd as moe
    from synth import configs

    tw = TOPK_WORKLOADS[args.workload]
    spec = configs.topk_rows_spec(args.workload)
    steps = args.steps or tw["steps"]
    warmup = tw["warmup"] if args.warmup is None else args.warmup
    n_copies = args.copies or tw["copies"]
    rows, n, k = spec["rows"], spec["n"], spec["k"]
    torch.cuda.init()
    moe.load()
    hip = Hip()
    t_gen = time.perf_counter()
    host = configs.gen_indexer_scores(spec)
    first = torch.from_numpy(host).cuda()
    copies = [first] + [first.clone() for _ in range(n_copies - 1)]
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    t_gen = time.perf_counter() - t_gen
    stream = torch.cuda.current_stream().cuda_stream

    def step(i, events=None):
        moe.moe_topk_rows(copies[i % n_copies], k, idx, vals, stream=stream, events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    w0 = time.perf_counter()
    hip.record(e0, stream)
    for i in range(steps):
        step(warmup + i)
    hip.record(e1, stream)
    hip.sync(e1)
    wall = time.perf_counter() - w0
    total_ms = hip.ms(e0, e1)
    # the same steps again with the dispatch's own timestamps
    ev = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(steps):
        step(warmup + i, events=(ctypes.c_void_p * 2)(ev[i][0].value, ev[i][1].value))
    torch.cuda.synchronize()
    kern_us = float(np.mean([hip.ms(a, b) for a, b in ev])) * 1e3
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    hip.destroy(e0)
    hip.destroy(e1)
    alg_bytes = rows * n * 4.0 + rows * k * 8.0
    achieved = alg_bytes / (kern_us * 1e-6) / 1e9
    threads = 1024 if n > 512 * 32 else 512  # workgroup size of the launch (one row per workgroup)
    out = {
        "metric": "row top-k rows/s (indexer selection); kernel HBM GB/s vs MI355X peak",
        "value": round(rows * steps / (total_ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(total_ms / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; indexer-shaped scores: head-weighted ReLU sums)",
        "config": {"workload": "%s: %d rows x %d candidates, top-%d, fp32 scores (%d copies rotated)"
                               % (args.workload, rows, n, k, n_copies),
                   "rows": rows, "n": n, "k": k, "workgroup_threads": threads},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": topk_traffic_record(args.workload),
                     "kernel": "topk_rows_kernel", "bytes_per_launch": alg_bytes, "avg_launch_us": round(kern_us, 3)},
        "wall_ms_per_step": round(wall * 1e3 / steps, 5),
        "setup_s": round(t_gen, 1),
    }
    if args.copy_probe_mib:
        out["copy_probe_GBs"] = copy_probe(torch, hip, stream, args.copy_probe_mib)
        out["copy_probe_bytes"] = args.copy_probe_mib * (1 << 20)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_topk(spec, host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


TOPK_SOURCES = [_CSRC + f for f in ("topk_rows.hip", "topk_rows.h", "common.h", "kernels.h")]


def topk_traffic_record(workload):
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(rec_path):
        return None
    with open(rec_path) as f:
        r = json.load(f).get(workload)
    if not r or r.get("kernel") != "topk_rows_kernel" or r.get("source_sha") != source_sha(TOPK_SOURCES):
        return None
    return r.get("hbm_bytes_per_launch")


def cpu_baseline_topk(spec, host, target_s=12.0):
    """The oracle's row top-k on a bounded sample of the workload's rows."""
    from oracle import Oracle
    orc = Oracle()
    n_rows, cap = 1, host.shape[0]

    def run(m):
        t0 = time.perf_counter()
        orc.topk_rows(host[:m], spec["k"])
        return time.perf_counter() - t0

    dt = run(n_rows)
    while dt < target_s / 2 and n_rows < cap:
        n_rows = int(min(cap, max(2 * n_rows, n_rows * target_s / max(dt, 1e-3))))
        dt = run(n_rows)
    reps = 1
    if dt < target_s / 2:  # the whole workload is quick: repeat it
        reps = int(target_s / 2 / max(dt, 1e-3)) + 1
        dt = sum(run(n_rows) for _ in range(reps))
    threads = orc.threads()
    return {"value": n_rows * reps / dt, "unit": "rows/s", "cores": min(threads, n_rows), "kind": "oracle",
            "sample": "%d rows of the workload per call, %d call(s) (sort-based oracle, one row per OpenMP "
                      "thread, %d threads), %.2f s wall" % (n_rows, reps, threads, dt)}


def dtype_of(cfg):
    """The arithmetic the layer's expert kernels compute in."""
    return {"q8b32": "int8xbf16", "bf16": "bf16", "f32": "f32"}[cfg["w"]]


DTYPE_NOTE = {
    "int8xbf16": "int8 weights in blocks of 32 with an fp16 scale, dequantised exactly in registers, times bf16 "
                 "activations; fp32 accumulation; router fp32 weights with fp64 accumulation",
    "bf16": "bf16 weights and activations on the bf16 matrix cores, fp32 accumulation; router fp32 weights with "
            "fp64 accumulation",
    "f32": "fp32 weights and activations, fp32 accumulation",
}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, L, x_all, target_s=12.0):
    """The oracle, as it stands, on a bounded sample of the workload, on all the
    host threads it was built for (OpenMP over tokens) and on one thread: the
    sample grows (from 8 tokens, or 1 on one thread, as the last call's rate
    suggests) until one call takes at least half of its target; that call is
    reported.  One thread gets a third of ``target_s``."""
    import numpy as np
    from oracle import Oracle
    orc = Oracle()
    threads = orc.threads()

    def run(n):
        Ls = dict(L)
        Ls["x"] = np.ascontiguousarray(x_all[:n])
        t0 = time.perf_counter()
        orc.layer_forward(cfg, Ls, debug=False)
        return time.perf_counter() - t0

    def grow(n, target):
        cap = x_all.shape[0]
        dt = run(n)
        while dt < target / 2 and n < cap:
            n = int(min(cap, max(2 * n, n * target / max(dt, 1e-3))))
            dt = run(n)
        return n, dt

    n, dt = grow(min(8, x_all.shape[0]), target_s)
    prev = orc.set_threads(1)
    try:
        n1, dt1 = grow(1, target_s / 3)
    finally:
        orc.set_threads(prev)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d tokens of the same workload in one call (token-major fp64 oracle, %d OpenMP threads),"
                      " %.1f s wall" % (n, threads, dt),
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": "%d tokens in one call, %.1f s wall" % (n1, dt1)},
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=sorted(WORKLOADS) + sorted(TOPK_WORKLOADS) + sorted(HOT_WORKLOADS),
                    help="one workload alone; default: c5 as the headline with the c2 decode layer beside it")
    ap.add_argument("--no-decode", action="store_true", help="default run: leave out the c2 decode section")
    ap.add_argument("--copies", type=int, default=None, help="weight copies rotated across steps")
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per step instead of the workload's (small-batch sweeps)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"],
                    help="force the decode (GEMV) or prefill (grouped GEMM) path")
    ap.add_argument("--graph", action="store_true",
                    help="capture the steps in a HIP graph (64 steps per graph) and replay it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefetch-wg", type=int, default=256, help="look-ahead: workgroups of the prefetch launch")
    ap.add_argument("--prefetch-rows", type=int, default=512,
                    help="look-ahead: leading rows of each matrix the prefetch reads (0: all)")
    ap.add_argument("--prefetch-which", type=int, default=3,
                    help="look-ahead: matrices the prefetch reads (bit 0 gate, 1 up, 2 down)")
    ap.add_argument("--stage-times", default="auto", choices=["auto", "live", "pass"],
                    help="take the gate/up kernel's times in the timed steps (live; the other stages always come "
                         "from a second eager pass) or every stage's in that pass (pass); auto: live for prefill, "
                         "pass for decode, whose 50 us steps the per-dispatch "
                         "timestamps would slow")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv "
                         "files of a run made with --copy-probe-mib")
    return ap.parse_args(argv)


def main():
    args = parse_args()
    if args.record_traffic:
        wl = args.workload or "c5"
        if wl in TOPK_WORKLOADS:
            record_traffic(wl, None, None, args.record_traffic[0], args.record_traffic[1],
                           (args.copy_probe_mib or 1024) * (1 << 20))
            return
        from synth import configs as _cf
        from sparse_moe_layer_02_amd.binding import DECODE_MAX_TOKENS
        spec = WORKLOADS[wl]
        cfg = _cf.get(spec["base"], T=args.tokens or spec["T"], **spec.get("over", {}))
        dec = args.path == "decode" or (args.path == "auto" and cfg["T"] <= DECODE_MAX_TOKENS)
        record_traffic(wl, "decode" if dec else "prefill", cfg["w"], args.record_traffic[0],
                       args.record_traffic[1], (args.copy_probe_mib or 1024) * (1 << 20), rpe=rows_per_expert(cfg))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE layer runs on a single MI355X "
              "(expert-parallel sharding across GPUs is not built); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.workload in TOPK_WORKLOADS:
        return bench_topk_rows(args)
    if args.workload in HOT_WORKLOADS:
        print(json.dumps(measure_hot(args)), flush=True)
        return
    if args.workload is not None:
        out = measure_layer(args, args.workload, args.steps, args.warmup, not args.no_cpu_baseline)
        print(json.dumps(out), flush=True)
        return
    # Default: the largest configuration (c5, 4096-token skewed prefill) is the
    # headline line; the c2 decode layer is measured in the same process after
    # it (its own step count and weight copies) and carried under "decode".
    out = measure_layer(args, "c5", args.steps, args.warmup, not args.no_cpu_baseline)
    if not args.no_decode:
        dec = measure_layer(args, "c2", None, None, not args.no_cpu_baseline)
        keep = ("value", "unit", "steps", "warmup", "ms_per_step", "per_step_ms", "dtype", "dtype_note", "config",
                "roofline", "layer_hbm_GBs", "layer_hbm_frac", "layer_bytes", "layer_roofline_frac",
                "expert_union_mean", "stages_us", "cpu_baseline")
        out["decode"] = {key: dec[key] for key in keep if key in dec}
    print(json.dumps(out), flush=True)


def measure_hot(args):
    """The grouped gate/up and down GEMMs over the rows c5 routes to its
    hottest experts (moe_route, then moe_permute of the masked assignments,
    then moe_expert_ffn timed alone): matrix-core TFLOP/s of those expert
    groups.  The kernels are the 256-row-tile ones c5 itself runs."""
    import numpy as np
    import torch
    from synth import configs
    import sparse_moe_layer_02_amd as moe

    spec = HOT_WORKLOADS[args.workload]
    steps = args.steps or spec["steps"]
    warmup = spec["warmup"] if args.warmup is None else args.warmup
    cfg = configs.get(spec["base"])
    T, E, k, d, F = cfg["T"], cfg["E"], cfg["k"], cfg["d"], cfg["F"]
    torch.cuda.init()
    moe.load()
    hip = Hip()
    L = gen_weights_host(dict(cfg, n_shared=0))
    for key in ("s_gate", "s_up", "s_down"):
        L[key] = None
    W = upload_copies(L, 1, torch)[0]
    x = configs.gen_x(cfg)
    x_dev = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    c = moe.config_from(dict(cfg, n_shared=0))
    ws = moe.workspace(c)
    stream = torch.cuda.current_stream().cuda_stream
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, x_dev, W["w_router"], W["bias"], None, idx, tw, ws, stream=stream)
    counts = torch.bincount(idx.flatten().long(), minlength=E)
    hot = torch.topk(counts, spec["hot"]).indices
    idx_h = torch.where(torch.isin(idx, hot.to(torch.int32)), idx, torch.full_like(idx, -1))
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    moe.moe_permute(c, idx_h, offsets, perm, inv, ws, stream=stream)
    slot_out = torch.empty((T * k, d), dtype=torch.float32, device="cuda")
    Wm = moe.make_weights(W)
    rows = int(counts[hot].sum().item())
    hot_rows = sorted((int(v) for v in counts[hot].tolist()), reverse=True)

    def ffn():
        moe.moe_expert_ffn(c, x_dev, Wm, offsets, perm, tw, slot_out, None, ws, stream=stream)

    for _ in range(warmup):
        ffn()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(steps):
        ffn()
    hip.record(e1, stream)
    hip.sync(e1)
    ms = hip.ms(e0, e1) / steps
    flops = 2.0 * rows * d * 3 * F
    tfs = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "matrix-core TFLOP/s of the grouped expert GEMMs on c5's hottest experts",
        "value": round(tfs, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "dtype": "bf16",
        "dtype_note": DTYPE_NOTE["bf16"],
        "data": "synthetic (seeded counter-based generator; random-init weights of the layer's shape)",
        "config": {"workload": "%s: the grouped gate/up and down GEMMs over the rows of c5's %d most-loaded "
                               "experts (c5's own routing), no shared expert" % (args.workload, spec["hot"]),
                   "T": T, "d_model": d, "n_expert": E, "top_k": k, "d_ff": F, "hot_experts": spec["hot"],
                   "hot_rows": rows, "hot_share": round(rows / float(T * k), 4), "rows_per_hot_expert": hot_rows},
        "mfma_frac": round(tfs / BF16_PEAK_TFS, 4),
        "flops_per_step": flops,
        "note": "gate/up and down launches together; profiles/ splits them by kernel",
    }


def measure_layer(args, wname, steps, warmup, with_cpu):
    """One layer workload: warm-up, the timed steps (one pair of events around
    all of them), the per-stage kernel times, a pass with an event between
    steps for the per-step distribution, and the oracle on the host cores."""
    import numpy as np
    import torch
    import sparse_moe_layer_02_amd as moe
    from synth import configs

    spec = WORKLOADS[wname]
    steps = steps or spec["steps"]
    warmup = spec["warmup"] if warmup is None else warmup
    cfg = configs.get(spec["base"], T=args.tokens or spec["T"], **spec.get("over", {}))
    T = cfg["T"]
    decode = args.path == "decode" or (args.path == "auto" and T <= moe.DECODE_MAX_TOKENS)
    n_copies = args.copies or spec["copies"]
    torch.cuda.init()
    moe.load()
    hip = Hip()

    t_gen = time.perf_counter()
    L = gen_weights_host(cfg)
    copies = upload_copies(L, n_copies, torch)
    la = bool(spec.get("lookahead"))
    if la and (T != 1 or args.graph or not decode):
        raise SystemExit("the look-ahead workload runs one token per step on the decode path, eagerly")
    if la:
        x_all = configs.gen_x_walk(cfg, N_DECODE_TOKENS, configs.LOOKAHEAD_RHO)
    elif T <= moe.DECODE_MAX_TOKENS:
        x_all = configs.gen_x(cfg, N_DECODE_TOKENS, stream=configs.S_DECODE)
    else:
        x_all = configs.gen_x(cfg)
    x_dev = torch.from_numpy(x_all.view(np.int16) if x_all.dtype == np.uint16 else x_all).cuda()
    t_gen = time.perf_counter() - t_gen

    c = moe.config_from(cfg, path=args.path)
    ws = moe.workspace(c)
    y = torch.empty((T, cfg["d"]), dtype=torch.float32, device="cuda")
    Wc = [moe.make_weights(cp) for cp in copies]
    stream = torch.cuda.current_stream().cuda_stream
    n_tok_rows = x_dev.shape[0]

    # router look-ahead (on while la_on[0]): the side stream routes this step's
    # token with the next step's router (inputs only: no wait), and reads the
    # predicted experts of the next step's weights once the step has ended
    # (one event per step, recorded without a system-scope fence)
    side = torch.cuda.Stream() if la else None
    side_ws = moe.workspace(c) if la else None
    pred = torch.empty((T, cfg["k"]), dtype=torch.int32, device="cuda") if la else None
    pred_w = torch.empty((T, cfg["k"]), dtype=torch.float32, device="cuda") if la else None
    la_ev = [hip.sync_event() for _ in range(warmup + steps)] if la else None
    la_on = [False]

    def hold(ms):
        """Queue a bounded spin kernel of about ms milliseconds on the stream, so
        that the host enqueues the steps behind it and its launch time (the
        look-ahead adds six runtime calls per step) stays out of the timed region."""
        if not la:
            return
        a0, a1 = hip.event(), hip.event()
        hip.record(a0, stream)
        torch.cuda._sleep(1 << 20)
        hip.record(a1, stream)
        hip.sync(a1)
        per = hip.ms(a0, a1) / float(1 << 20)
        torch.cuda._sleep(int(min(ms / max(per, 1e-9), 1 << 40)))

    def step(i, events=None, dbg=None, strm=None):
        r = (i * T) % n_tok_rows if n_tok_rows > T else 0
        st = stream if strm is None else strm
        moe.moe_layer_forward(c, x_dev[r:r + T], Wc[i % n_copies], y, ws, debug=dbg,
                              stream=st, stage_events=events)
        if la_on[0]:
            ev_e = la_ev[i % len(la_ev)]
            hip.record(ev_e, st)
            nxt = copies[(i + 1) % n_copies]
            moe.moe_route(c, x_dev[r:r + T], nxt["w_router"], nxt["bias"], None, pred, pred_w, side_ws,
                          stream=side.cuda_stream)
            hip.wait(side.cuda_stream, ev_e)
            moe.moe_prefetch_experts(c, Wc[(i + 1) % n_copies], pred, which=args.prefetch_which,
                                     rows=args.prefetch_rows, workgroups=args.prefetch_wg,
                                     stream=side.cuda_stream)

    la_off = None
    if la:  # the same steps without the look-ahead first
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        a0, a1 = hip.event(), hip.event()
        hold(0.2 * steps)
        hip.record(a0, stream)
        for i in range(steps):
            step(warmup + i)
        hip.record(a1, stream)
        hip.sync(a1)
        la_off = hip.ms(a0, a1) / steps
        la_on[0] = True

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        G = 64
        steps = max(G, (steps + G - 1) // G * G)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                step(i, strm=side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(G):
                step(warmup + i, strm=cap)
        graph.replay()
        torch.cuda.synchronize()

    # ---- timed region ----------------------------------------------------
    # Eager steps carry per-stage kernel events (the dispatches' own start and
    # end timestamps) and log the selected experts; graph replays carry none,
    # so their stage times come from an eager pass afterwards.
    stage_names = moe.binding.DECODE_STAGES if decode else moe.binding.STAGES
    stage_ids = [moe.binding.STAGES.index(n) for n in stage_names]
    n_ev = moe.binding.STAGE_EVENTS
    live = graph is None and (args.stage_times == "live" or (args.stage_times == "auto" and not decode))
    # Live: only the gate/up launch (the roofline kernel) carries its events
    # in the timed steps (each timed event's cache fence holds the next
    # dispatch by several microseconds); every stage's events come from a
    # second eager pass of the same steps, which also logs the selected
    # experts.  Default events: with the system-scope fence turned off, the
    # start timestamp moved ahead of the dispatch (a 163 us launch read 177).
    gu = moe.binding.STAGES.index("gate_up")
    gu_ev = [(hip.event(), hip.event()) for _ in range(steps)] if live else None
    gu_arr = [(ctypes.c_void_p * n_ev)(*[(p[0].value if j == 2 * gu else p[1].value if j == 2 * gu + 1 else None)
                                         for j in range(n_ev)]) for p in gu_ev] if live else None
    ev = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    ev_arr = [(ctypes.c_void_p * n_ev)(*[e.value for e in row]) for row in ev]
    idx_log = torch.empty((steps, T, cfg["k"]), dtype=torch.int32, device="cuda")
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    hold(0.2 * steps)
    hip.record(e0, stream)
    if graph is not None:
        for _ in range(steps // 64):
            graph.replay()
    elif live:
        for i in range(steps):
            step(warmup + i, events=gu_arr[i])
    else:
        for i in range(steps):
            step(warmup + i)
    hip.record(e1, stream)
    hip.sync(e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = hip.ms(e0, e1)
    ms_per_step = total_ms / steps

    # the same steps again, eagerly, for the stage times and the expert log
    for i in range(steps):
        step(warmup + i, events=ev_arr[i], dbg={"topk_idx": idx_log[i]})
    torch.cuda.synchronize()
    # a stage whose kernels the path does not launch has unrecorded events
    # and is left out; live, the gate/up time is the timed steps' own
    stage_ms = np.full((steps, len(stage_names)), np.nan)
    for i in range(steps):
        for col, sid in enumerate(stage_ids):
            if live and sid == gu:
                v = hip.ms_or_none(gu_ev[i][0], gu_ev[i][1])
            else:
                v = hip.ms_or_none(ev[i][2 * sid], ev[i][2 * sid + 1])
            stage_ms[i, col] = np.nan if v is None else v
    for row in ev + (gu_ev or []):
        for e in row:
            hip.destroy(e)
    stages_us = {name: round(float(stage_ms[:, col].mean()) * 1e3, 2) for col, name in enumerate(stage_names)
                 if not np.isnan(stage_ms[:, col]).any()}

    # ---- per-step distribution: the same steps with an event between steps --
    sev = [hip.event() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    hold(0.2 * steps)
    hip.record(sev[0], stream)
    for i in range(steps):
        step(warmup + i)
        hip.record(sev[i + 1], stream)
    hip.sync(sev[-1])
    per_step = np.array([hip.ms(sev[i], sev[i + 1]) for i in range(steps)])
    for e in sev:
        hip.destroy(e)

    # ---- algorithmic work -------------------------------------------------
    idx_np = idx_log.cpu().numpy()
    unions = np.array([len(np.unique(idx_np[i])) for i in range(steps)])
    n_exp = unions.astype(np.float64) + cfg["n_shared"]       # experts whose weights a step must read
    router_bytes = cfg["E"] * cfg["d"] * 4
    act_bytes = 2 if cfg["act"] == "bf16" else 4
    layer_bytes = n_exp * expert_bytes(cfg) + router_bytes + T * cfg["d"] * (act_bytes + 4)
    if decode:  # the routed gate/up launch; the shared expert's gate/up runs beside the router
        gu_bytes = unions.astype(np.float64) * expert_bytes(cfg, 2)
        flops_gu = 2.0 * T * cfg["k"] * cfg["d"] * 2 * cfg["F"]
    else:  # routed + shared gate/up; the GEMM also reads the gathered rows of x and writes h
        gu_bytes = (n_exp * expert_bytes(cfg, 2) + T * cfg["d"] * act_bytes
                    + (T * cfg["k"] + T * cfg["n_shared"]) * cfg["F"] * act_bytes)
        flops_gu = 2.0 * (T * cfg["k"] + T * cfg["n_shared"]) * cfg["d"] * 2 * cfg["F"]
    layer_flops = 2.0 * (T * cfg["k"] + T * cfg["n_shared"]) * cfg["d"] * 3 * cfg["F"]
    gu_us = stages_us["gate_up"]
    achieved = float(np.mean(gu_bytes)) / (gu_us * 1e-6) / 1e9
    path_kind = "decode" if decode else "prefill"
    traffic = traffic_record(path_kind, cfg["w"], wname, rows_per_expert(cfg))
    # the gate/up launch's own roofline: HBM time of its algorithmic bytes
    # against matrix-core time of its flops (bf16 peak), whichever is longer
    mfma_bound = spec.get("bound") == "mfma" or (
        not decode and cfg["w"] == "bf16" and flops_gu / (BF16_PEAK_TFS * 1e12) > float(np.mean(gu_bytes)) / (HBM_PEAK_GBS * 1e9))
    if mfma_bound:
        tfs = flops_gu / (gu_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_PEAK_TFS, "unit": "TFLOP/s",
                    "frac": round(tfs / BF16_PEAK_TFS, 4), "traffic": traffic,
                    "kernel": dominant(path_kind, cfg["w"], rows_per_expert(cfg))[0], "flops_per_launch": flops_gu,
                    "bytes_per_launch": float(np.mean(gu_bytes)), "avg_launch_us": gu_us}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": dominant(path_kind, cfg["w"], rows_per_expert(cfg))[0], "bytes_per_launch": float(np.mean(gu_bytes)),
                    "avg_launch_us": gu_us}

    value = T * steps / (total_ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_of(cfg), "dtype_note": DTYPE_NOTE[dtype_of(cfg)],
        "data": "synthetic (seeded counter-based generator; random-init weights of the layer's shape)",
        "config": {"workload": describe(cfg), "T": T, "d_model": cfg["d"], "n_expert": cfg["E"],
                   "top_k": cfg["k"], "d_ff": cfg["F"], "weights": cfg["w"], "activations": cfg["act"],
                   "path": path_kind, "weight_copies": n_copies, "hip_graph": bool(args.graph),
                   "stage_times": ("gate/up in the timed steps, the other stages in a second eager pass" if live
                                   else "second eager pass"),
                   "distinct_tokens": n_tok_rows if decode else T, "router_lookahead": la},
        "roofline": roofline,
        "layer_hbm_GBs": round(float(np.mean(layer_bytes)) / (ms_per_step * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(float(np.mean(layer_bytes)) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_bytes": float(np.mean(layer_bytes)),
        "layer_roofline_frac": round(max(float(np.mean(layer_bytes)) / (HBM_PEAK_GBS * 1e9),
                                         (layer_flops / (BF16_PEAK_TFS * 1e12)) if cfg["w"] == "bf16" else 0.0)
                                     / (ms_per_step * 1e-3), 4),
        "per_step_ms": {"p50": round(float(np.percentile(per_step, 50)), 5),
                        "p90": round(float(np.percentile(per_step, 90)), 5),
                        "min": round(float(per_step.min()), 5), "max": round(float(per_step.max()), 5),
                        "note": "a separate eager pass of the same steps with an event between consecutive steps"},
        "expert_union_mean": float(unions.mean()),
        "stages_us": stages_us,
        "gate_up_tflops": round(flops_gu / (gu_us * 1e-6) / 1e12, 2),
        "wall_ms_per_step": round(wall * 1e3 / steps, 5),
        "setup_s": round(t_gen, 1),
    }
    if not decode:
        out["mfma_frac_gate_up"] = round(out["gate_up_tflops"] / BF16_PEAK_TFS, 4)
    if la:
        # copies share the router weights, so the next step's prediction (its
        # router on this step's token) is this step's own selection
        hits = [len(set(idx_np[i].ravel()) & set(idx_np[i + 1].ravel())) / cfg["k"] for i in range(steps - 1)]
        out["lookahead"] = {
            "rho": configs.LOOKAHEAD_RHO, "hit_rate": round(float(np.mean(hits)), 4),
            "off_value": round(T / (la_off * 1e-3), 2), "off_ms_per_step": round(la_off, 5),
            "gain": round(ms_per_step and la_off / ms_per_step, 4),
            "prefetch_workgroups": args.prefetch_wg, "prefetch_which": args.prefetch_which,
            "prefetch_rows": args.prefetch_rows,
            "enqueue": "both passes queued behind a bounded spin kernel (host launch time outside the timed region)"}

    if args.copy_probe_mib:
        out["copy_probe_GBs"] = copy_probe(torch, hip, stream, args.copy_probe_mib)
        out["copy_probe_bytes"] = args.copy_probe_mib * (1 << 20)

    # ---- the oracle on the host cores -----------------------------------
    out["cpu_baseline"] = cpu_baseline(cfg, L, x_all, args.cpu_seconds) if with_cpu else None
    del copies, Wc, x_dev, ws, L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
