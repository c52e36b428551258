#!/usr/bin/env python3
"""Decode-attention benchmark: batch 1, 64k context, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fd_decode call over the whole KV cache: B=1, Hq=64, Hkv=8,
D=128, 65536 cached tokens, bf16, scale 1/sqrt(128) -- the per-chunk pass
and, when the plan splits, the log-sum-exp merge.  Inputs are seeded
synthetic N(0,1) values (long_context_decode_fd_amd.workloads), resident in
HBM before timing starts.  Successive steps rotate over 4 copies of the KV
cache (1.07 GB) so that the 256 MB Infinity Cache cannot serve a repeat of
the previous step: each step reads its 268 MB from HBM, as a model's layers
do in turn.  W untimed steps (continued until at least 50 ms of warm-up, the
count reported as warmup_steps_run), then exactly K steps between two HIP
events on the launch stream with device synchronisation on both sides.

Prints one JSON line: value = algorithmic bytes per step (every K and V row
once, q, out, lse) / step time, in GB/s; the roofline object compares the
dominant kernel with MI355X's 8 TB/s HBM peak (and, as frac_of_stream_ceiling,
with stream_read_ceiling: a plain streaming read of the same number of bytes,
measured in the same run); cpu_baseline times the fp64 CPU oracle on the
host's cores over the same workload.  `configs` reports the five decode
workloads (tiny fp32 multi-head, batch-1 64k, batch-4 multi-head 32k with
peaked rows, batch-64 4k, variable-length batch of 16), each timed the
same way in the same run: µs/step, GB/s and fraction of 8 TB/s for the
whole step and for the per-chunk pass alone, and the plan.

--workload picks another workload of long_context_decode_fd_amd.workloads,
including the paged-cache (fd_decode_paged) and multi-token
(fd_decode_multiquery) ones; for those, as for --unified-max and
--fused-merge, the roofline object covers the whole step, since their
per-chunk pass has no separate phase call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode-attention µs/step and achieved HBM GB/s (% of peak), "
          "batch 1 @ 64k ctx")
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
KV_COPIES = 4
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_b1_gqa8_64k.json")
KERNEL_SRC = os.path.join(ROOT, "long_context_decode_fd_amd", "csrc",
                          "fd_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Untimed warm-up runs at least this long whatever W is: MI355X reaches its
# steady step time only after some milliseconds of continuous work (20
# steps: 47.8 us/step; 200 or more: 46.5).
MIN_WARMUP_S = 0.05


def warm_up(torch, fn, steps: int) -> int:
    """Runs fn(i) for `steps` steps, then more until MIN_WARMUP_S of
    device time has passed; returns the number of steps run."""
    i = 0
    t0 = time.perf_counter()
    while i < steps:
        fn(i)
        i += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(50):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def stream_ceiling(torch, nbytes: int, steps: int, warmup: int, stream):
    """Practical HBM read ceiling: libfdprobe.so's plain streaming read of
    nbytes, rotating over KV_COPIES buffers like the decode steps, timed
    the same way (HIP events on the launch stream)."""
    import ctypes
    from long_context_decode_fd_amd import build as lib_build
    if not os.path.exists(lib_build.PROBE_LIB):
        raise RuntimeError(f"{lib_build.PROBE_LIB} not built: run "
                           "python -m long_context_decode_fd_amd.build")
    lib = ctypes.CDLL(lib_build.PROBE_LIB)
    lib.fdp_stream_read.restype = ctypes.c_int
    lib.fdp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    n = nbytes // 16 * 16
    bufs = [torch.full((n,), 1 + i, dtype=torch.uint8, device="cuda")
            for i in range(KV_COPIES)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = ctypes.c_void_p(stream.cuda_stream)

    def rd(i):
        rc = lib.fdp_stream_read(bufs[i % KV_COPIES].data_ptr(), n,
                                 sink.data_ptr(), 256, h)
        if rc != 0:
            raise RuntimeError(f"fdp_stream_read failed: {rc}")

    for i in range(warmup):
        rd(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        rd(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    del bufs
    return {"GBs": n / (us * 1e-6) / 1e9, "us": us, "bytes": n,
            "kernel": "stream_read (long_context_decode_fd_amd/csrc/"
                      "fd_probe.hip), 256 workgroups, 16-byte nontemporal "
                      f"loads, {KV_COPIES} rotated buffers"}


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel source with comments and whitespace
    removed: counters stay valid across comment-only edits and become
    stale with any change of the code."""
    import re
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = "".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(PMC_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if doc.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since counters were taken"
    return doc.get("hbm_bytes_per_launch"), doc.get("kernel")


SAMPLE_KV_BYTES = 1 << 30     # host-side K/V of the CPU baseline's sample


def cpu_baseline(w, budget_s: float):
    """fp64 oracle over the same workload on the host's cores: whole steps
    of the first batch entries whose K/V fit SAMPLE_KV_BYTES (all of them
    for the batch-1 workloads), repeated until ~budget_s of wall time (at
    least one run); the rate is taken from the median run.  A one-thread
    time of the same sample (at most 3 runs or ~budget_s / 4) is added."""
    import numpy as np
    from long_context_decode_fd_amd import workloads as wl
    from oracle import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    per_b = 2 * w.Hkv * w.Lmax * w.D * w.elem_bytes
    nb = max(1, min(w.B, SAMPLE_KV_BYTES // per_b))
    # The generator's streams are per slab, and q / seqlens are drawn in
    # batch order, so the first nb entries of the workload are exactly the
    # workload with B = nb (a paged sample gets its own page table).
    ws = w.with_(B=nb)
    q, k, v, seqlens = wl.gen_all(ws)
    if w.page_size:
        seqlens = wl.paged_seqlens(ws, seqlens)
        bt = wl.gen_block_table(ws)
        kp, vp = wl.scatter_pages(ws, k, v, bt, seqlens)
        del k, v

        def run(n):
            oracle.decode_paged(q, kp, vp, bt, seqlens, w.scale, nthreads=n)
    elif w.Tq > 1:
        def run(n):
            oracle.decode_multiquery(q, k, v, seqlens, w.scale, nthreads=n)
    else:
        def run(n):
            oracle.decode(q, k, v, seqlens, w.scale, nthreads=n)

    def timed(n, budget, max_runs):
        ts = []
        t_total = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            run(n)
            ts.append(time.perf_counter() - t0)
            if time.perf_counter() - t_total >= budget or len(ts) >= max_runs:
                return ts

    times = timed(cores, budget_s, 1000)
    t = float(np.median(times))
    # one thread as well (per-core figure), a few runs at most
    times1 = timed(1, budget_s / 4, 3)
    t1 = float(np.median(times1))
    nbytes = wl.algorithmic_bytes(ws, seqlens)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": nbytes / t / 1e9, "unit": "GB/s", "cores": cores,
        "kind": "oracle", "us_per_step": t * 1e6,
        "one_thread": {"us_per_step": t1 * 1e6,
                       "value": nbytes / t1 / 1e9, "runs": len(times1)},
        "sample": (f"{len(times)} run(s) over batch entries 0..{nb - 1} of "
                   f"{w.B} (all {w.Hq} query heads, same inputs as the GPU "
                   f"run), median wall time, rate = their algorithmic bytes "
                   f"/ time; fp64 C oracle, OpenMP over rows, {cores} "
                   f"threads" + (f", {model}" if model else "")
                   + ("; the sample's own page table" if w.page_size
                      else "")),
    }


def timed_us(torch, fn, steps: int, warmup: int, stream) -> float:
    """Average µs of fn(i) over `steps` calls between two HIP events on
    `stream`, after warm_up(warmup) and a device synchronisation."""
    warm_up(torch, fn, warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


GRAPH_STEPS = 20    # decode calls per captured graph


def graph_us(torch, call, steps: int, warmup: int) -> float:
    """Device time per call: GRAPH_STEPS calls call(i) captured in one HIP
    graph (the calls must queue kernels only), the graph replayed until
    steps calls have run, between two HIP events; no host work between
    the kernels, so short steps are not limited by the Python caller."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(GRAPH_STEPS):
            call(i)
    torch.cuda.synchronize()
    reps = max(1, steps // GRAPH_STEPS)
    stream = torch.cuda.current_stream()
    warm_up(torch, lambda i: g.replay(), max(1, warmup // GRAPH_STEPS))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * GRAPH_STEPS) * 1e3


def config_table(torch, fd, wl, steps: int, warmup: int, stream) -> dict:
    """The five decode workloads, each timed the same way in this run.

    Per workload: the whole fd_decode step (planner's plan, KV rotated over
    KV_COPIES copies when one copy is under 1 GB, so that the 256 MB
    Infinity Cache cannot serve a repeat; larger caches exceed it alone),
    algorithmic bytes / step time against 8 TB/s, and for split plans the
    per-chunk pass alone (fd_decode_partials, same plan) with its bytes
    (K, V, q) / time.  A single-pass plan (no merge) is its own per-chunk
    pass.  us_per_step_graph is the same step replayed from a HIP graph
    (fd_decode_ex with a caller workspace: the same plan and kernels),
    which takes the Python caller out of the measurement.  The tiny fp32
    workload is latency-bound: its fraction of peak is not a bandwidth
    figure."""
    table = {}
    for name in wl.WORKLOAD_ORDER:
        w = wl.WORKLOADS[name]
        log(f"[bench] config {name}: generating inputs")
        q, k, v, sl, seqlens, _ = wl.device_inputs(w)
        kv_bytes = 2 * k.numel() * k.element_size()
        copies = KV_COPIES if kv_bytes < (1 << 30) else 1
        ks = [k] + [k.clone() for _ in range(copies - 1)]
        vs = [v] + [v.clone() for _ in range(copies - 1)]
        out = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                          varlen=sl is not None)
        step_us = timed_us(torch, lambda i: fd.fd_decode(
            q, ks[i % copies], vs[i % copies], sl, w.scale, out=out,
            lse=lse, stream=stream), steps, warmup, stream)
        ws = torch.empty(max(plan["workspace_bytes"], 256),
                         dtype=torch.uint8, device="cuda")
        step_graph_us = graph_us(torch, lambda i: fd.fd_decode_ex(
            q, ks[i % copies], vs[i % copies], sl, w.scale, out=out,
            lse=lse, workspace=ws), steps, warmup)
        del ws
        nbytes = wl.algorithmic_bytes(w, seqlens)
        io_bytes = w.B * w.Hq * w.D * w.elem_bytes + 4 * w.B * w.Hq
        row = {
            "us_per_step": step_us,
            "us_per_step_graph": step_graph_us,
            "GBs": nbytes / step_us / 1e3,
            "frac_of_peak": nbytes / step_us / 1e3 / PEAK_HBM_GBS,
            "algorithmic_bytes": nbytes,
            "kv_copies_rotated": copies,
            "plan": {"num_splits": plan["num_splits"],
                     "chunk": plan["chunk"], "grid": plan["grid"],
                     "variant": "mfma" if plan["variant"] ==
                     fd.FD_VARIANT_MFMA else "valu",
                     "merge_pass": bool(plan["combine"])},
        }
        if plan["combine"]:
            pplan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                               varlen=sl is not None,
                               flags=fd.FD_FLAG_PARTIALS)
            ws = torch.zeros(pplan["workspace_bytes"], dtype=torch.uint8,
                             device="cuda")
            kern_us = timed_us(torch, lambda i: fd.fd_decode_partials(
                q, ks[i % copies], vs[i % copies], sl, w.scale, ws,
                stream=stream), steps, warmup, stream)
            kern_graph_us = graph_us(torch, lambda i: fd.fd_decode_partials(
                q, ks[i % copies], vs[i % copies], sl, w.scale, ws),
                steps, warmup)
            kbytes = nbytes - io_bytes
            row["per_chunk_pass"] = {
                "us": kern_us, "us_graph": kern_graph_us,
                "GBs": kbytes / kern_us / 1e3,
                "frac_of_peak": kbytes / kern_us / 1e3 / PEAK_HBM_GBS,
                "bytes": kbytes}
            del ws
        else:
            row["per_chunk_pass"] = {
                "us": step_us, "us_graph": step_graph_us, "GBs": row["GBs"],
                "frac_of_peak": row["frac_of_peak"], "bytes": nbytes,
                "note": "single-pass plan: the step is the per-chunk pass"}
        if w.dtype == "f32":
            row["note"] = ("latency-bound (4 MB per step): report the µs; "
                           "the fraction of peak is not a bandwidth figure")
        log(f"[bench] config {name}: {step_us:.2f} us/step "
            f"({step_graph_us:.2f} from a graph), "
            f"{row['frac_of_peak'] * 100:.1f}% of 8 TB/s, per-chunk pass "
            f"{row['per_chunk_pass']['us']:.2f} us")
        table[name] = row
        del q, k, v, ks, vs, out, lse
        torch.cuda.empty_cache()
    return table


def context_sweep(torch, fd, steps: int) -> None:
    """Flash-Decoding against the same kernel unsplit, over context length.

    [FD], section "A faster attention for decoding: Flash-Decoding", compares
    splitting the keys/values with attention that parallelises over batch
    and heads only, which at small batch leaves most of the GPU idle.  Here
    the unsplit form is this library's own kernel with num_splits = 1 (one
    workgroup per (sequence, KV head)); the split form is the planner's
    plan.  Batch 1 and 8, 64 query heads on 8 KV heads, D = 128, bf16,
    seeded random inputs, KV rotated over KV_COPIES copies.  Each form is
    timed from a HIP graph (device time per step: at short contexts an
    eager Python call costs more host time than the step takes on the GPU)
    and eagerly through fd_decode / fd_decode_ex.  One JSON line per case.
    """
    D, Hq, Hkv = 128, 64, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    stream = torch.cuda.current_stream()
    for B in (1, 8):
        for L in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072):
            if B * L > 8 * 65536:
                continue
            shape = (B, Hkv, L, D)
            ks = [torch.randn(shape, device="cuda", dtype=torch.bfloat16,
                              generator=gen) for _ in range(KV_COPIES)]
            vs = [torch.randn(shape, device="cuda", dtype=torch.bfloat16,
                              generator=gen) for _ in range(KV_COPIES)]
            q = torch.randn((B, Hq, D), device="cuda", dtype=torch.bfloat16,
                            generator=gen)
            out = torch.empty_like(q)
            lse = torch.empty((B, Hq), device="cuda")
            scale = D ** -0.5
            plan = fd.fd_plan(B, Hq, Hkv, D, L, "bf16")
            ws = torch.empty(max(plan["workspace_bytes"], 256),
                             dtype=torch.uint8, device="cuda")
            res = {"sweep": "split_vs_unsplit", "B": B, "L": L, "Hq": Hq,
                   "Hkv": Hkv, "D": D, "num_splits": plan["num_splits"],
                   "chunk": plan["chunk"]}
            for tag, S in (("split", 0), ("unsplit", 1)):
                def call(i, S=S):
                    fd.fd_decode_ex(q, ks[i % KV_COPIES], vs[i % KV_COPIES],
                                    None, scale, out=out, lse=lse,
                                    num_splits=S, workspace=ws)
                res[f"{tag}_us"] = round(graph_us(torch, call, steps,
                                                  steps), 2)
                res[f"{tag}_us_eager"] = round(
                    timed_us(torch, call, steps, steps, stream), 2)
            nbytes = 2 * B * Hkv * L * D * 2
            res["speedup"] = round(res["unsplit_us"] / res["split_us"], 2)
            res["split_GBs"] = round(nbytes / res["split_us"] / 1e3, 1)
            res["unsplit_GBs"] = round(nbytes / res["unsplit_us"] / 1e3, 1)
            print(json.dumps(res), flush=True)
            del ks, vs, ws
            torch.cuda.empty_cache()


SPLIT_SWEEP_SHAPES = [  # (B, Hq, Hkv, D, dtype)
    (1, 64, 8, 128, "bf16"), (2, 64, 8, 128, "bf16"), (4, 64, 8, 128, "bf16"),
    (8, 32, 8, 128, "bf16"), (16, 32, 8, 128, "bf16"),
    (1, 32, 32, 128, "bf16"), (4, 32, 32, 128, "bf16"),
    (1, 8, 8, 64, "f32"), (4, 8, 8, 64, "f32"), (1, 64, 8, 128, "f32")]
SPLIT_SWEEP_LENGTHS = (256, 384, 512, 768, 1024, 1536, 2048, 4096, 8192,
                       16384, 32768)


def split_sweep(torch, fd, steps: int) -> None:
    """The planner's split count against every split count from 1 to 128,
    over batch, head layout and context length: device time per step from
    a HIP graph (fd_decode_ex with forced num_splits and a caller
    workspace; the faster of two measurements), KV rotated over up to 8
    copies so that the working set of short caches exceeds the 256 MB
    Infinity Cache.  One JSON line per
    shape: the planner's choice, every split count's time, the fastest."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    for B, Hq, Hkv, D, dtype in SPLIT_SWEEP_SHAPES:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        for L in SPLIT_SWEEP_LENGTHS:
            if dtype == "f32" and L > 4096:
                continue
            shape = (B, Hkv, L, D)
            kvb = 2 * B * Hkv * L * D * (2 if dtype == "bf16" else 4)
            copies = max(1, min(8, (1 << 30) // kvb))
            ks = [torch.randn(shape, device="cuda", dtype=tdt,
                              generator=gen) for _ in range(copies)]
            vs = [torch.randn(shape, device="cuda", dtype=tdt,
                              generator=gen) for _ in range(copies)]
            q = torch.randn((B, Hq, D), device="cuda", dtype=tdt,
                            generator=gen)
            out = torch.empty_like(q)
            lse = torch.empty((B, Hq), device="cuda")
            scale = D ** -0.5
            auto = fd.fd_plan(B, Hq, Hkv, D, L, dtype)
            res = {"sweep": "split_count", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "D": D, "dtype": dtype, "L": L,
                   "planner": [auto["num_splits"], auto["chunk"]]}
            n = steps if kvb < (32 << 20) else max(40, steps // 4)
            for S in (1, 2, 4, 8, 16, 32, 64, 128):
                if S > L // 32 or B * Hkv * S > 8192:
                    continue
                p = fd.fd_plan(B, Hq, Hkv, D, L, dtype, num_splits=S)
                ws = torch.empty(max(p["workspace_bytes"], 256),
                                 dtype=torch.uint8, device="cuda")

                def call(i, S=S, ws=ws):
                    fd.fd_decode_ex(q, ks[i % copies], vs[i % copies], None,
                                    scale, out=out, lse=lse, num_splits=S,
                                    workspace=ws)
                # the faster of two measurements: single device-time
                # figures on a shared box can catch a slow spell
                res[f"S{p['num_splits']}"] = round(min(
                    graph_us(torch, call, n, n // 2) for _ in range(2)), 2)
            if f"S{auto['num_splits']}" not in res:
                ws = torch.empty(max(auto["workspace_bytes"], 256),
                                 dtype=torch.uint8, device="cuda")
                res[f"S{auto['num_splits']}"] = round(min(graph_us(
                    torch, lambda i: fd.fd_decode_ex(
                        q, ks[i % copies], vs[i % copies], None, scale,
                        out=out, lse=lse, workspace=ws), n, n // 2)
                    for _ in range(2)), 2)
            times = {k: v for k, v in res.items() if k[0] == "S"}
            res["fastest"] = min(times, key=times.get)
            res["planner_over_fastest"] = round(
                times[f"S{auto['num_splits']}"] / times[res["fastest"]], 3)
            print(json.dumps(res), flush=True)
            del ks, vs
            torch.cuda.empty_cache()


def fused_sweep(torch, fd, steps: int) -> None:
    """The single-launch merge (FD_FLAG_FUSED_MERGE) against the separate
    merge pass over the split-sweep shapes and 256-32768 keys: device time
    per step from a HIP graph (fd_decode_ex with a caller workspace whose
    tickets start at zero; the faster of two measurements), the separate
    merge at the planner's split count, the fused one at that count, half
    and a quarter of it.  One JSON line per shape."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    F = fd.FD_FLAG_FUSED_MERGE
    for B, Hq, Hkv, D, dtype in SPLIT_SWEEP_SHAPES:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        for L in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            if dtype == "f32" and L > 4096:
                continue
            shape = (B, Hkv, L, D)
            kvb = 2 * B * Hkv * L * D * (2 if dtype == "bf16" else 4)
            copies = max(1, min(8, (1 << 30) // kvb))
            ks = [torch.randn(shape, device="cuda", dtype=tdt,
                              generator=gen) for _ in range(copies)]
            vs = [torch.randn(shape, device="cuda", dtype=tdt,
                              generator=gen) for _ in range(copies)]
            q = torch.randn((B, Hq, D), device="cuda", dtype=tdt,
                            generator=gen)
            out = torch.empty_like(q)
            lse = torch.empty((B, Hq), device="cuda")
            scale = D ** -0.5
            S0 = fd.fd_plan(B, Hq, Hkv, D, L, dtype)["num_splits"]
            n = steps if kvb < (32 << 20) else max(40, steps // 4)

            def timed(S, flags):
                p = fd.fd_plan(B, Hq, Hkv, D, L, dtype, num_splits=S,
                               flags=flags)
                ws = torch.zeros(max(p["workspace_bytes"], 256),
                                 dtype=torch.uint8, device="cuda")

                def call(i):
                    fd.fd_decode_ex(q, ks[i % copies], vs[i % copies], None,
                                    scale, out=out, lse=lse, num_splits=S,
                                    flags=flags, workspace=ws)
                return round(min(graph_us(torch, call, n, n // 2)
                                 for _ in range(2)), 2)
            res = {"sweep": "fused_merge", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "D": D, "dtype": dtype, "L": L, "planner_splits": S0,
                   "separate": timed(S0, 0)}
            if S0 > 1:
                for S in sorted({S0, max(2, S0 // 2), max(2, S0 // 4)},
                                reverse=True):
                    res[f"fused_S{S}"] = timed(S, F)
            print(json.dumps(res), flush=True)
            del ks, vs
            torch.cuda.empty_cache()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--workload", default=None,
                    help="another workload of long_context_decode_fd_amd."
                         "workloads (default: the batch-1 64k one)")
    ap.add_argument("--unified-max", type=float, default=None, metavar="PHI",
                    help="time fd_decode_unified_max with this phi instead "
                         "of fd_decode (contiguous single-token workloads)")
    ap.add_argument("--context-sweep", action="store_true",
                    help="instead of the benchmark line: Flash-Decoding "
                         "against the same kernel unsplit over context "
                         "length (batch 1 and 8), one JSON line per case")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table of the five decode "
                         "workloads")
    ap.add_argument("--fused-merge", action="store_true",
                    help="time fd_decode_ex with FD_FLAG_FUSED_MERGE (the "
                         "single-launch merge) instead of fd_decode "
                         "(contiguous single-token workloads)")
    ap.add_argument("--split-sweep", action="store_true",
                    help="instead of the benchmark line: the planner's split "
                         "count against split counts 1..128 over batch, "
                         "heads and context length, one JSON line per shape")
    ap.add_argument("--fused-sweep", action="store_true",
                    help="instead of the benchmark line: the single-launch "
                         "merge against the separate merge pass over the "
                         "same shapes, one JSON line per shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter "
                         "runs: HBM bytes per counter unit)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(the decode path has no multi-GPU form in this library)",
              file=sys.stderr)
        return 2

    import torch
    import long_context_decode_fd_amd as fd
    from long_context_decode_fd_amd import workloads as wl

    if a.context_sweep or a.split_sweep or a.fused_sweep:
        torch.cuda.set_device(0)
        fd.load_library()
        if a.context_sweep:
            context_sweep(torch, fd, a.steps)
        if a.split_sweep:
            split_sweep(torch, fd, a.steps)
        if a.fused_sweep:
            fused_sweep(torch, fd, a.steps)
        return 0

    w = wl.ALL_WORKLOADS[a.workload or wl.BENCH_WORKLOAD]
    kind = ("paged" if w.page_size else
            "multiquery" if w.Tq > 1 else
            "unified_max" if a.unified_max is not None else
            "fused" if a.fused_merge else "decode")
    torch.cuda.set_device(0)
    fd.load_library()
    log(f"[bench] workload {w.name} ({kind}): generating inputs")
    stream = torch.cuda.current_stream()
    if kind == "paged":
        q, k, v, bt, sl, seqlens, _ = wl.device_paged_inputs(w)
        plan = fd.fd_plan_ex(w.B, w.Tq, w.Hq, w.Hkv, w.D,
                             w.max_pages * w.page_size, w.dtype, paged=True)
    else:
        q, k, v, sl, seqlens, _ = wl.device_inputs(w)
        plan = fd.fd_plan_ex(w.B, w.Tq, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                             varlen=sl is not None,
                             flags=fd.FD_FLAG_UNIFIED_MAX
                             if kind == "unified_max" else
                             fd.FD_FLAG_FUSED_MERGE if kind == "fused" else 0)
    # the fused merge's tickets start at zero and every call leaves them so
    fused_ws = (torch.zeros(max(plan["workspace_bytes"], 256),
                            dtype=torch.uint8, device="cuda")
                if kind == "fused" else None)
    ks = [k] + [k.clone() for _ in range(KV_COPIES - 1)]
    vs = [v] + [v.clone() for _ in range(KV_COPIES - 1)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def call(kk, vv):
        if kind == "paged":
            fd.fd_decode_paged(q, kk, vv, bt, sl, w.scale, out=out, lse=lse,
                               head_major=w.head_major, stream=stream)
        elif kind == "multiquery":
            fd.fd_decode_multiquery(q, kk, vv, sl, w.scale, out=out, lse=lse,
                                    stream=stream)
        elif kind == "unified_max":
            fd.fd_decode_unified_max(q, kk, vv, sl, w.scale, a.unified_max,
                                     out=out, lse=lse, stream=stream)
        elif kind == "fused":
            fd.fd_decode_ex(q, kk, vv, sl, w.scale, out=out, lse=lse,
                            flags=fd.FD_FLAG_FUSED_MERGE, workspace=fused_ws,
                            stream=stream)
        else:
            fd.fd_decode(q, kk, vv, sl, w.scale, out=out, lse=lse,
                         stream=stream)

    def step(i):
        call(ks[i % KV_COPIES], vs[i % KV_COPIES])

    # The same step with a caller workspace (the same plan and kernels),
    # for replay from a HIP graph: device time without the Python caller.
    gws = torch.zeros(max(plan["workspace_bytes"], 256), dtype=torch.uint8,
                      device="cuda") if kind != "fused" else fused_ws

    def call_ws(kk, vv):
        if kind == "paged":
            fd.fd_decode_paged(q, kk, vv, bt, sl, w.scale, out=out, lse=lse,
                               head_major=w.head_major, workspace=gws)
        elif kind == "multiquery":
            fd.fd_decode_multiquery(q, kk, vv, sl, w.scale, out=out, lse=lse,
                                    workspace=gws)
        elif kind == "unified_max":
            fd.fd_decode_unified_max(q, kk, vv, sl, w.scale, a.unified_max,
                                     out=out, lse=lse, workspace=gws)
        else:
            fd.fd_decode_ex(q, kk, vv, sl, w.scale, out=out, lse=lse,
                            flags=fd.FD_FLAG_FUSED_MERGE if kind == "fused"
                            else 0, workspace=gws)

    log(f"[bench] plan {plan}")
    warmup_run = warm_up(torch, step, a.warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    th0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    host_us = (time.perf_counter() - th0) / a.steps * 1e6
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    log(f"[bench] timed {a.steps} steps: {ms * 1e3:.2f} us/step")

    # Spread of the step time: BLOCKS more blocks of BLOCK_STEPS rotated
    # steps, each between two HIP events; median and min of their means.
    BLOCKS, BLOCK_STEPS = 10, 20
    block_us = []
    for blk in range(BLOCKS):
        e0.record(stream)
        for i in range(BLOCK_STEPS):
            step(blk * BLOCK_STEPS + i)
        e1.record(stream)
        torch.cuda.synchronize()
        block_us.append(e0.elapsed_time(e1) / BLOCK_STEPS * 1e3)
    block_us.sort()

    # Same-buffer ("hot") figure, labelled as such: repeats may hit MALL.
    e0.record(stream)
    for i in range(a.steps):
        call(k, v)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_hot = e0.elapsed_time(e1) / a.steps

    step_graph_us = graph_us(torch, lambda i: call_ws(ks[i % KV_COPIES],
                                                       vs[i % KV_COPIES]),
                             a.steps, a.warmup)
    log(f"[bench] the same steps replayed from a graph: "
        f"{step_graph_us:.2f} us/step")

    kern_avg_ms = None
    if kind == "decode":
        # Dominant kernel on its own: the per-chunk pass of the same plan
        # (fd_decode_partials), K launches back to back between two HIP
        # events on the launch stream, then one merge to leave out/lse
        # consistent.
        pplan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                           varlen=sl is not None, flags=fd.FD_FLAG_PARTIALS)
        assert (pplan["num_splits"], pplan["chunk"], pplan["grid"]) == \
            (plan["num_splits"], plan["chunk"], plan["grid"])
        ws = torch.zeros(pplan["workspace_bytes"], dtype=torch.uint8,
                         device="cuda")
        warm_up(torch, lambda i: fd.fd_decode_partials(
            q, ks[i % KV_COPIES], vs[i % KV_COPIES], sl, w.scale, ws,
            stream=stream), a.warmup)
        e0.record(stream)
        for i in range(a.steps):
            fd.fd_decode_partials(q, ks[i % KV_COPIES], vs[i % KV_COPIES],
                                  sl, w.scale, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        kern_avg_ms = e0.elapsed_time(e1) / a.steps
        fd.fd_merge_partials(sl, w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype, ws,
                             out, lse, stream=stream)
        torch.cuda.synchronize()

    ceiling = stream_ceiling(torch, wl.algorithmic_bytes(w, seqlens), a.steps,
                             a.warmup, stream)
    log(f"[bench] streaming-read ceiling {ceiling['GBs']:.0f} GB/s")

    if a.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = wl.algorithmic_bytes(w, seqlens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    split_kernel = (f"split_mfma_kernel<{w.D}, {plan['waves_per_block']}, "
                    f"{'paged' if kind == 'paged' else 'contiguous'}"
                    f"{', unified max' if kind == 'unified_max' else ''}"
                    f"{', fused merge' if kind == 'fused' else ''}>"
                    if plan["variant"] == fd.FD_VARIANT_MFMA else
                    f"split_valu_kernel<{w.dtype}, {w.D}>")
    if kern_avg_ms is not None:
        # The per-chunk pass must read every K/V row and q once; out/lse
        # are the merge pass's.
        kbytes = nbytes - (w.B * w.Hq * w.D * w.elem_bytes + 4 * w.B * w.Hq)
        kgbs = kbytes / (kern_avg_ms * 1e-3) / 1e9
        traffic, traffic_note = (traffic_from_profiles()
                                 if w.name == wl.BENCH_WORKLOAD
                                 else (None, "counters taken for the batch-1 "
                                             "64k workload only"))
        roof = {
            "bound": "hbm", "achieved": kgbs, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": kgbs / PEAK_HBM_GBS, "traffic": traffic,
            "kernel": f"{split_kernel} (per-chunk pass)",
            "bytes_per_launch": kbytes,
            "avg_launch_us": kern_avg_ms * 1e3,
            "timing": f"{a.steps} back-to-back launches of the per-chunk "
                      "pass (fd_decode_partials, same plan) between two HIP "
                      f"events on the launch stream, KV rotated over "
                      f"{KV_COPIES} copies",
            "traffic_note": traffic_note,
        }
    else:
        roof = {
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None,
            "kernel": f"{split_kernel} + merge (whole step)",
            "bytes_per_launch": nbytes, "avg_launch_us": ms * 1e3,
            "timing": f"{a.steps} whole steps between two HIP events on the "
                      f"launch stream, KV rotated over {KV_COPIES} copies; "
                      "this layout has no separate per-chunk phase call",
            "traffic_note": "counters taken for the batch-1 64k workload "
                            "only",
        }
    res = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup,
        "warmup_steps_run": warmup_run, "ms_per_step": ms,
        "us_per_step": ms * 1e3, "frac_of_peak": gbs / PEAK_HBM_GBS,
        "us_per_step_graph": step_graph_us,
        "host_us_per_call": host_us,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic (seeded N(0,1) {w.dtype} q/K/V)",
        "config": {"workload": w.name, "call": "fd_decode" if kind == "decode"
                   else "fd_decode_ex (FD_FLAG_FUSED_MERGE)" if kind == "fused"
                   else f"fd_decode_{kind}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "seq_len": w.Lmax, "Tq": w.Tq,
                   "page_size": w.page_size, "unified_max_phi": a.unified_max,
                   "page_layout": ("head-major" if w.head_major else
                                   "token-major") if w.page_size else None,
                   "kv_copies_rotated": KV_COPIES,
                   "num_splits": plan["num_splits"], "chunk": plan["chunk"],
                   "grid": plan["grid"], "waves_per_block":
                   plan["waves_per_block"], "merge_pass": bool(plan["combine"])},
        "step_spread": {"blocks": BLOCKS, "steps_per_block": BLOCK_STEPS,
                        "median_us": block_us[BLOCKS // 2],
                        "min_us": block_us[0], "max_us": block_us[-1],
                        "note": "means of separately timed blocks of "
                                "rotated steps, after the timed region"},
        "hot_same_buffer": {"us_per_step": ms_hot * 1e3,
                            "GBs": nbytes / (ms_hot * 1e-3) / 1e9,
                            "note": "one KV copy re-read every step; may be "
                                    "served partly from the 256 MB MALL"},
        "roofline": roof,
        "stream_read_ceiling": ceiling,
    }
    roof["frac_of_stream_ceiling"] = roof["achieved"] / ceiling["GBs"]
    if (not a.no_configs and a.workload is None and a.unified_max is None
            and not a.fused_merge):
        del ks, vs, k, v
        torch.cuda.empty_cache()
        res["configs"] = config_table(torch, fd, wl, a.steps, a.warmup,
                                      stream)
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle")
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
