#!/usr/bin/env python3
"""Throughput of the PATCH hybrid tile-sparse GEMM on one MI355X.

PATCH (arXiv 2509.23410): every 128 x 128 tile of W is dense or 2:4 sparse
(gist.science explainer, section 2 "Core Mechanism"); the pages report only
end-to-end numbers (1.18x-1.38x over dense, LLaMA-2 7B on an A6000, section 4
"Speedup & Efficiency"), so there is no published kernel figure to compare
with and vs_baseline is null.

Default workload (the headline line): the LLaMA-2-7B MLP prefill GEMMs --
gate/up 11008 x 4096 and down 4096 x 11008, bf16, 2202 of their 2752
128 x 128 tiles 2:4 (40% sparsity), top-2-of-4 masks, X of 2048 tokens.
One step = one patch_gemm on each matrix (the hybrid GEMM with its
epilogue; packing is offline and timed separately).  Inputs are resident in
HBM; every launch reads its own copy of the packed weight (>= 1 GiB rotated
per matrix) so the 256 MB Infinity Cache cannot serve them.  The line also
carries the decode workload (q_proj 4096 x 4096, M = 1, 4, 16), a sparsity
sweep on three shapes, ceilings measured in the same run and the CPU
oracle's rate.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--report out.jsonl]

Prints one JSON line.  --report also writes the sweep over all workloads
(every sparse-tile fraction, decode and prefill shapes) as JSON lines.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 matrix peak, datasheet
ROTATE_BYTES = 1 << 30          # >= 1 GiB of distinct weights per timed loop
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# --hybrid-only: time the hybrid launches alone (no dense, all-dense-packed or
# hipBLASLt references; the headline without its graph-replay figure), so
# that a profiler's per-kernel figures cover the headline's timed launches
# alone -- the all-dense packed reference runs the same kernels
HYBRID_ONLY = False
# Untimed settle phase before every timed measurement: the calls are repeated
# back to back for this long first.  From idle, the GPU's power management
# takes some 20-40 ms of sustained load to settle; launches timed before that
# ran up to 25% slower (the prefill MLP step: 0.34 ms in its first 14 ms, then
# 0.29-0.30 ms).  --settle-ms sets it.
SETTLE_MS = 150.0
KERNEL_SOURCES = ("sparse_gemm_amd/csrc/gemm_decode.hip", "sparse_gemm_amd/csrc/gemm_prefill.hip",
                  "sparse_gemm_amd/csrc/prefill_common.h", "sparse_gemm_amd/csrc/device_common.h")


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def blob_bytes(N, K, n_sparse):
    T = (N // 128) * (K // 128)
    return -(-(256 + 16 * T) // 256) * 256 + 32768 * (T - n_sparse) + 18432 * n_sparse


def algo_bytes(N, K, M, n_sparse, packed=True):
    w = blob_bytes(N, K, n_sparse) if packed else 2 * N * K
    return w + 2 * M * K + 2 * M * N


def dev_bits(bits, torch_dtype):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_dtype).cuda()


def _event():
    import torch

    e = torch.cuda.Event(enable_timing=True)
    e.record()
    return e


def settle(calls, ms=None):
    """Untimed: run the calls back to back (launch index k * len(calls) + c,
    so the weight copies keep rotating) until `ms` of host time has passed,
    synchronising every few steps so the GPU is busy for about that long."""
    import torch

    ms = SETTLE_MS if ms is None else ms
    if ms <= 0:
        return
    n, k = len(calls), 0
    t_end = time.perf_counter() + ms * 1e-3
    while time.perf_counter() < t_end:
        for c, (_, fn) in enumerate(calls):
            fn(k * n + c)
        k += 1
        if k % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_launches(calls, steps, warmup, batches=1):
    """calls: list of (key, fn(i)); fn(i) issues launch i of that call (it
    picks its weight copy from i).  Returns
      * ms per step, a step running every call once, back to back (one event
        pair around all `steps` steps; step k gives call c the index
        (warmup + k) * len(calls) + c, so no two launches of a step share a
        copy), and
      * {key: [ms per launch of each batch]}, each call timed on its own:
        `batches` batches of `steps` launches back to back (indices warmup,
        warmup + 1, ...), one event pair around each batch, divided by
        `steps`.
    Events are recorded on the current stream, the one the launches use.
    An untimed settle phase (settle()) comes first."""
    import torch

    settle(calls)
    n = len(calls)
    for k in range(warmup):
        for c, (_, fn) in enumerate(calls):
            fn(k * n + c)
    torch.cuda.synchronize()
    a = _event()
    for k in range(steps):
        for c, (_, fn) in enumerate(calls):
            fn((warmup + k) * n + c)
    b = _event()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    per = {}
    for key, fn in calls:
        for k in range(warmup):
            fn(k)
        per[key] = []
        for _ in range(batches):
            a = _event()
            for k in range(steps):
                fn(warmup + k)
            b = _event()
            torch.cuda.synchronize()
            per[key].append(a.elapsed_time(b) / steps)
    return ms_step, per


def time_steps(calls, steps, warmup):
    """The timed region of the headline: `steps` steps, each running every
    call once (call c of step k gets index (warmup + k) * len(calls) + c),
    issued back to back on the current stream between one pair of HIP
    events.  Returns ms per step.  An untimed settle phase (settle()) and
    `warmup` untimed steps come first."""
    import torch

    settle(calls)
    n = len(calls)
    for k in range(warmup):
        for c, (_, fn) in enumerate(calls):
            fn(k * n + c)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(steps):
        for c, (_, fn) in enumerate(calls):
            fn((warmup + k) * n + c)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_steps_events(calls, steps, warmup):
    """The timed region of the headline: `steps` steps, each running every
    call once (call c of step k gets index (warmup + k) * len(calls) + c),
    issued back to back on the current stream with a HIP event recorded
    before every launch and one after the last.  Returns ms per step (first
    to last event / steps) and {key: [ms of each of its launches]} (event to
    next event), so the launches' durations add up to the step time exactly.
    Every launch here is long against its host cost, so the stream never
    waits for the host.  An untimed settle phase (settle()) comes first."""
    import torch

    settle(calls)
    n = len(calls)
    for k in range(warmup):
        for c, (_, fn) in enumerate(calls):
            fn(k * n + c)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps * n + 1)]
    i = 0
    for k in range(steps):
        for c, (_, fn) in enumerate(calls):
            evs[i].record()
            fn((warmup + k) * n + c)
            i += 1
    evs[i].record()
    torch.cuda.synchronize()
    per = {key: [] for key, _ in calls}
    for j in range(steps * n):
        per[calls[j % n][0]].append(evs[j].elapsed_time(evs[j + 1]))
    return evs[0].elapsed_time(evs[-1]) / steps, per


def _capture(fns):
    """One HIP graph that runs fns in order (each a no-argument launch on
    the current stream).  Every fn runs once eagerly first, on the capture
    side stream, so lazy set-up happens outside the graph."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns[: min(len(fns), 8)]:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graphs(calls, steps, warmup, batches=1):
    """As time_launches (same launch indices), but the launches are captured
    in HIP graphs and the graphs replayed, so host launch overhead is out of
    the timed region:
      * ms per step: one graph of `steps` steps (every call once a step, back
        to back), replayed once untimed and once between one event pair;
      * {key: [ms per launch of each batch]}: per call, one graph of `steps`
        launches, replayed `batches` times, each between one event pair.
    An untimed settle phase (settle()) comes first."""
    import torch

    settle(calls)
    n = len(calls)
    for k in range(warmup):
        for c, (_, fn) in enumerate(calls):
            fn(k * n + c)
    torch.cuda.synchronize()
    g = _capture([(lambda fn=fn, i=(warmup + k) * n + c: fn(i)) for k in range(steps)
                  for c, (_, fn) in enumerate(calls)])
    g.replay()
    torch.cuda.synchronize()
    a = _event()
    g.replay()
    b = _event()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    del g
    per = {}
    for key, fn in calls:
        g = _capture([(lambda k=k: fn(warmup + k)) for k in range(steps)])
        g.replay()
        torch.cuda.synchronize()
        per[key] = []
        for _ in range(batches):
            a = _event()
            g.replay()
            b = _event()
            torch.cuda.synchronize()
            per[key].append(a.elapsed_time(b) / steps)
        del g
    torch.cuda.empty_cache()
    return ms_step, per


def rotate(t, nbytes_each):
    """t and copies of it, >= ROTATE_BYTES in all (so the 256 MB Infinity
    Cache cannot hold them); the count is prime to 2 and 3, so launches that
    index the copies with a stride of 2 or 3 (a step's calls) still visit
    every copy."""
    n = max(5, min(65, int(np.ceil(ROTATE_BYTES / max(1, nbytes_each)))))
    while n % 2 == 0 or n % 3 == 0:
        n += 1
    return [t] + [t.clone() for _ in range(n - 1)]


_WS = {}


def ws_for(key, nbytes_fn):
    """The workspace of one call site (key), allocated on its first call --
    in the untimed settle phase that starts every timed region -- at the
    size the library asks for, then reused: the timed launches carry no
    allocator work, as in a serving loop or a captured graph."""
    import torch

    w = _WS.get(key)
    if w is None:
        w = _WS[key] = torch.empty(max(16, int(nbytes_fn())), dtype=torch.uint8, device="cuda")
    return w


def ws_gemm(desc, M):
    from sparse_gemm_amd import patch

    # keyed by what the size depends on (not by the descriptor object, whose
    # id a later one may reuse)
    return ws_for(("gemm", desc.version, desc.N, desc.K, M),
                  lambda: patch.load().patch_gemm_workspace_bytes(ctypes.byref(desc), M))


def ws_dense(M, N, K):
    from sparse_gemm_amd import patch

    return ws_for(("dense", M, N, K), lambda: patch.load().patch_dense_gemm_workspace_bytes(M, N, K))


def ws_swiglu(desc, M):
    from sparse_gemm_amd import patch

    return ws_for(("swiglu", desc.version, desc.N, desc.K, M),
                  lambda: patch.load().patch_gemm_swiglu_workspace_bytes(ctypes.byref(desc), M))


def pack_timed(W, tile_map, mask):
    import torch

    from sparse_gemm_amd import patch

    pw = patch.pack(W, tile_map, mask)  # warm-up (also the product)
    best = None
    for _ in range(3):
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        patch.pack(W, tile_map, mask, out=pw.blob)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    return pw, best


def gemm_set(cfg_name, mi, si, Ms, steps, warmup, with_hipblaslt=True, fraction=None, map_kind=None, batches=1):
    """Time patch_gemm, patch_dense_gemm and torch.matmul for one weight matrix."""
    import torch

    from sparse_gemm_amd import inputs, patch

    cfg = inputs.CONFIGS[cfg_name]
    p = inputs.make_weights(cfg, mi, si, fraction=fraction, map_kind=map_kind)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float16
    W = dev_bits(p.w, tdt)
    mask = torch.from_numpy(p.mask).cuda()
    pw, pack_ms = pack_timed(W, p.tile_map, mask)
    refs = not HYBRID_ONLY
    p0 = patch.pack(W, np.zeros_like(p.tile_map), mask) if refs else None  # the same weights, every tile dense
    del mask
    blobs = rotate(pw.blob, pw.nbytes)
    blobs0 = rotate(p0.blob, p0.nbytes) if refs else None
    Ws = rotate(W, W.numel() * 2)
    Xs = {M: dev_bits(inputs.make_x(cfg, M, p.K, matrix_index=mi), tdt) for M in Ms}
    Ys = {M: torch.empty((M, p.N), dtype=tdt, device="cuda") for M in Ms}
    desc = pw.desc

    # f(i): launch i on weight copy i mod the copies
    def hyb(M):
        def f(i):
            patch.gemm(Xs[M], patch.PackedWeight(blobs[i % len(blobs)], desc), out=Ys[M], workspace=ws_gemm(desc, M))
        return f

    def hyb0(M):
        def f(i):
            patch.gemm(Xs[M], patch.PackedWeight(blobs0[i % len(blobs0)], p0.desc), out=Ys[M],
                       workspace=ws_gemm(p0.desc, M))
        return f

    def dense(M):
        def f(i):
            patch.dense_gemm(Xs[M], Ws[i % len(Ws)], out=Ys[M], workspace=ws_dense(M, p.N, p.K))
        return f

    def blas(M):
        def f(i):
            torch.matmul(Xs[M], Ws[i % len(Ws)].t(), out=Ys[M])
        return f

    # our kernels: graph replays (launch overhead out of the timed region)
    # and eager back-to-back launches; hipBLASLt (torch.matmul): eager only,
    # since a library call may record work that graph replays do not repeat
    # faithfully
    ms_h, per_h = time_graphs([(M, hyb(M)) for M in Ms], steps, warmup, batches)
    ms_0 = per_0 = ms_d = per_d = per_b = None
    if refs:
        ms_0, per_0 = time_graphs([(M, hyb0(M)) for M in Ms], steps, warmup, batches)
        ms_d, per_d = time_graphs([(M, dense(M)) for M in Ms], steps, warmup, batches)
    ms_he, per_he = time_launches([(M, hyb(M)) for M in Ms], steps, warmup, batches)
    if with_hipblaslt and refs:
        _, per_b = time_launches([(M, blas(M)) for M in Ms], steps, warmup, batches)
    res = dict(p=p, pw=pw, pack_ms=pack_ms, ms_step=ms_h, ms_step_dense=ms_0, per=per_h, per_dense=per_0,
               ms_step_rowmajor=ms_d, per_rowmajor=per_d, ms_step_eager=ms_he, per_eager=per_he, per_blas=per_b,
               n_copies=len(blobs))
    del blobs, blobs0, Ws
    torch.cuda.empty_cache()
    return res


def mean(x):
    return float(np.mean(x))


def median(x):
    return float(np.median(x))


def summarize(res, Ms):
    p = res["p"]
    N, K, ns = p.N, p.K, int(p.tile_map.sum())
    T = p.tile_map.size
    s = ns / T
    out = {}
    for M in Ms:
        t = median(res["per"][M]) * 1e-3
        fl = 2.0 * M * N * K
        eff = 2.0 * M * N * K * (1 - 0.5 * s)
        e = dict(us=t * 1e6, us_min=min(res["per"][M]) * 1e3, us_max=max(res["per"][M]) * 1e3,
                 batches=len(res["per"][M]), us_eager=median(res["per_eager"][M]) * 1e3,
                 tflops_dense_equiv=fl / t / 1e12, tflops_effective=eff / t / 1e12,
                 gbps=algo_bytes(N, K, M, ns) / t / 1e9)
        if res["per_dense"] is not None:
            td = median(res["per_dense"][M]) * 1e-3  # the same weights packed all-dense, same kernels
            tr = median(res["per_rowmajor"][M]) * 1e-3  # patch_dense_gemm on row-major W
            e.update(dense_us=td * 1e6, speedup_vs_dense=td / t, rowmajor_dense_us=tr * 1e6,
                     speedup_vs_rowmajor_dense=tr / t)
        if res["per_blas"] is not None:
            # eager against eager: both include the host's launch cost
            tb = median(res["per_blas"][M]) * 1e-3
            e["hipblaslt_us_eager"] = tb * 1e6
            e["speedup_vs_hipblaslt_eager"] = tb / (e["us_eager"] * 1e-6)
        # roofline: max of HBM time and blended matrix-core time
        t_hbm = algo_bytes(N, K, M, ns) / (HBM_PEAK_GBS * 1e9)
        t_mma = 2.0 * M * 128 * 128 * ((T - ns) / MFMA_PEAK_BF16_TFLOPS + ns / (2 * MFMA_PEAK_BF16_TFLOPS)) / 1e12
        e["roofline_bound"] = "hbm" if t_hbm >= t_mma else "mfma"
        e["roofline_frac"] = max(t_hbm, t_mma) / t
        out[M] = e
    return out


def traffic_for(kernel, M):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the
    kernel sources are unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha") != kernel_sha():
        return None
    ent = d.get("kernels", {}).get(kernel, {}).get(str(M))
    if not ent:
        return None
    return float(ent["fetch_bytes"] + ent["write_bytes"])


def ingest_counters(dirs):
    """Write profiles/traffic_counters.json from rocprofv3 counter runs of this
    script with --calibrate-copy: dirs = [fetch_dir, write_dir, ...], pairs of
    one --pmc FETCH_SIZE run and one --pmc WRITE_SIZE run of the same command
    (CSV output).  Per-dispatch KiB are averaged per kernel and scaled by what
    the same counter reads for the 256 MiB device copy of known size in the
    same run."""
    import csv
    import glob

    if len(dirs) % 2:
        raise SystemExit("--ingest-counters takes FETCH_DIR WRITE_DIR pairs")

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                if "copyBuffer" in name:
                    key = "copy"
                elif "k_decode<" in name:
                    key = "decode_dense" if name.split("<")[1].split(",")[1].strip() == "true" else "decode"
                elif "k_prefill<" in name or "k_prefill_lds<" in name:
                    key = "prefill_dense" if name.split("<")[1].split(",")[1].strip() == "true" else "prefill"
                else:
                    continue
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    copy_kib = 256 * 1024.0
    kernels, scales = {}, []
    for fetch_dir, write_dir in zip(dirs[0::2], dirs[1::2]):
        fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
        # the copy reads and writes 256 MiB; take the largest copy dispatch (the calibration one)
        f_scale = copy_kib / max(fetch["copy"])
        w_scale = copy_kib / max(write["copy"])
        scales.append((f_scale, w_scale))
        for key in sorted(set(fetch) & set(write) - {"copy"}):
            fb = mean(fetch[key]) * 1024.0 * f_scale
            wb = mean(write[key]) * 1024.0 * w_scale
            Ms = (1, 4, 16) if key.startswith("decode") else (2048,)
            kernels[key] = {str(M): {"fetch_bytes": fb, "write_bytes": wb} for M in Ms}
            kernels[key]["raw_kib"] = {"fetch": mean(fetch[key]), "write": mean(write[key]),
                                       "dispatches": len(fetch[key])}
    out = {"kernel_sha": kernel_sha(),
           "note": "rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch, averaged over all dispatches of each kernel "
                   "in its run (decode: M = 1, 4, 16 launches alike; prefill: both matrices of the prefill MLP "
                   "workload), scaled by a 256 MiB device copy measured in the same run (fetch, write scales: " +
                   ", ".join(f"x{a:.4f} x{b:.4f}" for a, b in scales) + ")",
           "scales": scales, "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(problems, Ms, sample_rows, budget_s=10.0):
    """The oracle, as it stands, on a bounded sample of the same step: the
    first `sample_rows` rows of each call's X against the full weights
    (every output column, every tile), repeated for about `budget_s`
    seconds; reported as dense-equivalent TFLOP/s of the rows it did."""
    import oracle
    from sparse_gemm_amd import inputs

    work = []
    for (p, cfg, mi), M in zip(problems, Ms):
        rows = min(M, sample_rows)
        work.append((p, inputs.make_x(cfg, M, p.K, matrix_index=mi)[:rows], rows))
    flops = sum(2.0 * rows * p.N * p.K for p, _, rows in work)
    reps, t0 = 0, time.perf_counter()
    while True:
        for p, xb, _ in work:
            oracle.gemm_f64(p.dtype, xb, p.w, p.tile_map, p.mask)
        reps += 1
        el = time.perf_counter() - t0
        if el > budget_s or reps >= 5000:
            break
    desc = "; ".join(f"{rows} of {M} rows of X against the full {p.N}x{p.K} weight" for (p, _, rows), M in
                     zip(work, Ms))
    return dict(value=flops * reps / el / 1e12, unit="TFLOP/s (dense-equivalent)", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"{reps} repetition(s) of oracle_gemm_f64 (fp64, plain C) on a row sample of the step "
                       f"({desc}; same weights, tile maps and masks); {el:.1f} s wall")


def measure_ceilings(read_bytes, steps=20):
    """What one launch can reach on this device, measured in this run:
    streaming reads of each byte count in `read_bytes` (distinct buffers
    rotated past the Infinity Cache, as the GEMM weights are) and the
    sustained rate of each matrix instruction the kernels use."""
    import torch

    from sparse_gemm_amd import patch

    out = {"hbm_read": {}, "matrix_core_tflops": {}}
    sink = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    for nb in read_bytes:
        nb = int(nb) // 16 * 16
        bufs = rotate(torch.ones(nb, dtype=torch.uint8, device="cuda"), nb)
        _, per = time_graphs([("r", lambda i: patch.probe_stream_read(bufs[i % len(bufs)], sink))], steps, 5, 3)
        t = median(per["r"]) * 1e-3
        out["hbm_read"][str(nb)] = dict(us=t * 1e6, gbps=nb / t / 1e9, frac_of_peak=nb / t / 1e9 / HBM_PEAK_GBS)
        del bufs
        torch.cuda.empty_cache()
    names = {0: "mfma_f32_16x16x32_bf16", 1: "smfmac_f32_16x16x64_bf16", 2: "mfma_f32_32x32x16_bf16",
             3: "smfmac_f32_32x32x32_bf16"}
    wgs = 2 * 256  # two workgroups of four waves a CU
    for kind, name in names.items():
        flops = patch.probe_matrix_rate(kind, 64, wgs, sink)  # warm-up
        iters = 4000
        torch.cuda.synchronize()
        a = _event()
        flops = patch.probe_matrix_rate(kind, iters, wgs, sink)
        b = _event()
        torch.cuda.synchronize()
        out["matrix_core_tflops"][name] = flops / (a.elapsed_time(b) * 1e-3) / 1e12
    # global -> LDS copies (the prefill kernels' copy instruction and ring), one
    # workgroup of 8 waves a CU: 16 windows of 256 KB (held by the L2s after
    # the first pass) and one 512 KB window a workgroup (128 MB in all: past
    # the L2s, Infinity Cache resident)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.ones(256 * (512 << 10), dtype=torch.uint8, device="cuda")
    out["lds_copy_tbs"] = {}
    for name, nbytes, win, iters in (("l2_resident", 16 * (256 << 10), 256 << 10, 3000),
                                     ("past_l2", 256 * (512 << 10), 512 << 10, 3000)):
        view = src[:nbytes]
        patch.probe_copy_rate(view, win, 10, ncu, sink)  # warm-up (and first touch)
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            a = _event()
            nb = patch.probe_copy_rate(view, win, iters, ncu, sink)
            b = _event()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None or t < best else best
        out["lds_copy_tbs"][name] = nb / best / 1e12
    del src
    torch.cuda.empty_cache()
    out["note"] = ("hbm_read: patch_probe_stream_read over that many bytes (16-byte loads, one pass), median of 3 "
                   "graph replays of 20 launches on rotated buffers; matrix_core_tflops: patch_probe_matrix_rate, "
                   "2 workgroups of 4 waves a CU, independent accumulator chains, dense-equivalent flops for the "
                   "sparse instructions; lds_copy_tbs: patch_probe_copy_rate (global -> LDS with the prefill "
                   "kernels' copy instruction, 8 waves a CU, 7 KB a wave per iteration, two-slot ring), L2-resident "
                   "windows and windows past the L2s, best of 3; datasheet peaks: 8000 GB/s, 2516.6 TFLOP/s dense "
                   "bf16 (x2 with 2:4)")
    return out


def t_mfma_s(M, T, ns):
    """Matrix-core time of one launch at the blended datasheet peak: dense
    tiles at the dense bf16 peak, 2:4 tiles' dense-equivalent work at twice
    it (the sparse instruction's rate)."""
    return 2.0 * M * 128 * 128 * ((T - ns) / MFMA_PEAK_BF16_TFLOPS + ns / (2 * MFMA_PEAK_BF16_TFLOPS)) / 1e12


def eff_flops(M, T, ns):
    """Work the hybrid GEMM actually does: 32768 flop per token per dense
    tile, 16384 per 2:4 tile."""
    return 2.0 * M * 128 * 128 * ((T - ns) + 0.5 * ns)


def headline_prefill(args):
    """The prefill MLP workload (LLaMA-2-7B gate/up 11008 x 4096 and down
    4096 x 11008, bf16, 80% of tiles 2:4 (2202 of 2752), top-2-of-4 masks,
    X 2048 x K): one step = one hybrid GEMM on each matrix."""
    import torch

    from sparse_gemm_amd import inputs, patch

    cfg = inputs.CONFIGS["prefill_mlp"]
    M = cfg.Ms[0]
    mats = []
    for mi in range(len(cfg.matrices)):
        p = inputs.make_weights(cfg, mi, 0)
        W = dev_bits(p.w, torch.bfloat16)
        mk = torch.from_numpy(p.mask).cuda()
        pw, pack_ms = pack_timed(W, p.tile_map, mk)
        # the same weights with every tile dense
        p0 = patch.pack(W, np.zeros_like(p.tile_map), mk) if not HYBRID_ONLY else None
        del mk
        X = dev_bits(inputs.make_x(cfg, M, p.K, matrix_index=mi), torch.bfloat16)
        refs = p0 is not None
        mats.append(dict(name=cfg.matrices[mi].name, p=p, pw=pw, pack_ms=pack_ms, blobs=rotate(pw.blob, pw.nbytes),
                         blobs0=rotate(p0.blob, p0.nbytes) if refs else None, desc0=p0.desc if refs else None,
                         Ws=rotate(W, W.numel() * 2) if refs else None, X=X,
                         Y=torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda")))
        del p0, W

    def hyb(m):
        return lambda i: patch.gemm(m["X"], patch.PackedWeight(m["blobs"][i % len(m["blobs"])], m["pw"].desc),
                                    out=m["Y"], workspace=ws_gemm(m["pw"].desc, M))

    def hyb0(m):
        return lambda i: patch.gemm(m["X"], patch.PackedWeight(m["blobs0"][i % len(m["blobs0"])], m["desc0"]),
                                    out=m["Y"], workspace=ws_gemm(m["desc0"], M))

    def dense(m):
        return lambda i: patch.dense_gemm(m["X"], m["Ws"][i % len(m["Ws"])], out=m["Y"],
                                          workspace=ws_dense(M, m["p"].N, m["p"].K))

    def blas(m):
        return lambda i: torch.matmul(m["X"], m["Ws"][i % len(m["Ws"])].t(), out=m["Y"])

    steps, warmup = args.steps, args.warmup
    ms_step = time_steps([(m["name"], hyb(m)) for m in mats], steps, warmup)
    # the per-launch breakdown: the same steps with an event before every launch
    ms_step_ev, per = time_steps_events([(m["name"], hyb(m)) for m in mats], steps, warmup)
    ms_step_graph = None
    if not HYBRID_ONLY:
        ms_step_graph, _ = time_graphs([(m["name"], hyb(m)) for m in mats], steps, warmup)
    refs = not HYBRID_ONLY
    ms_dense = per_dense = ms_s0 = per_s0 = ms_blas = ms_blas_ev = per_blas = per_hb = per_bb = None
    if refs:
        ms_dense = time_steps([(m["name"], dense(m)) for m in mats], steps, warmup)
        ms_s0 = time_steps([(m["name"], hyb0(m)) for m in mats], steps, warmup)
        ms_blas = time_steps([(m["name"], blas(m)) for m in mats], steps, warmup)
        _, per_dense = time_steps_events([(m["name"], dense(m)) for m in mats], steps, warmup)
        _, per_s0 = time_steps_events([(m["name"], hyb0(m)) for m in mats], steps, warmup)
        ms_blas_ev, per_blas = time_steps_events([(m["name"], blas(m)) for m in mats], steps, warmup)
        # like for like against the library: batches of back-to-back launches
        # between one event pair, no event between launches (an event between
        # two torch.matmul launches costs them more than it costs ours)
        _, per_hb = time_launches([(m["name"], hyb(m)) for m in mats], steps, warmup, 3)
        _, per_bb = time_launches([(m["name"], blas(m)) for m in mats], steps, warmup, 3)

    def ref_us(per_ref, name):
        return mean(per_ref[name]) * 1e3 if refs else None

    def ref_speedup(per_ref, name, t):
        return mean(per_ref[name]) * 1e-3 / t if refs else None

    flops_step = sum(2.0 * M * m["p"].N * m["p"].K for m in mats)
    per_matrix = {}
    eff_sum, t_sum, n_launch, tm_sum = 0.0, 0.0, 0, 0.0
    for m in mats:
        p = m["p"]
        T, ns = int(p.tile_map.size), int(p.tile_map.sum())
        t = mean(per[m["name"]]) * 1e-3
        tm = t_mfma_s(M, T, ns)
        per_matrix[m["name"]] = dict(
            N=p.N, K=p.K, M=M, sparse_tiles=ns, tiles=T, us=t * 1e6, us_min=min(per[m["name"]]) * 1e3,
            us_max=max(per[m["name"]]) * 1e3, tflops_dense_equiv=2.0 * M * p.N * p.K / t / 1e12,
            tflops_effective=eff_flops(M, T, ns) / t / 1e12, roofline_us=tm * 1e6, roofline_frac=tm / t,
            dense_us=ref_us(per_s0, m["name"]),
            rowmajor_dense_us=ref_us(per_dense, m["name"]),
            hipblaslt_us=median(per_bb[m["name"]]) * 1e3 if refs else None,
            hybrid_us_batched=median(per_hb[m["name"]]) * 1e3 if refs else None,
            hipblaslt_us_events=ref_us(per_blas, m["name"]),
            speedup_vs_dense=ref_speedup(per_s0, m["name"], t),
            speedup_vs_rowmajor_dense=ref_speedup(per_dense, m["name"], t),
            speedup_vs_hipblaslt=median(per_bb[m["name"]]) / median(per_hb[m["name"]]) if refs else None,
            speedup_vs_hipblaslt_events=ref_speedup(per_blas, m["name"], t),
            pack_us=m["pack_ms"] * 1e3, pack_gbps=(3 * p.N * p.K + m["pw"].nbytes) / (m["pack_ms"] * 1e-3) / 1e9,
            weight_copies_rotated=len(m["blobs"]))
        eff_sum += eff_flops(M, T, ns)
        tm_sum += tm
        n_launch += 1
    # the roofline's launch time: the headline's step time (one event pair
    # over the K steps) over the step's launches
    avg_t = ms_step * 1e-3 / n_launch
    achieved = eff_sum / (ms_step * 1e-3) / 1e12
    traffic = traffic_for("prefill", M)
    line = {
        "metric": "hybrid GEMM TFLOP/s (dense-equiv) + speedup vs dense, LLaMA-2-7B shapes",
        "value": flops_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) X, N(0,0.02) W; LLaMA-2-7B MLP shapes, no weights)",
        "config": {
            "workload": "prefill_mlp: LLaMA-2-7B MLP GEMMs gate/up 11008x4096 and down 4096x11008, bf16, "
                        "2202 of 2752 128x128 tiles 2:4 (40% sparsity), top-2-of-4 masks, X 2048 tokens; "
                        "one step = patch_gemm on each of the two matrices",
            "M": M, "matrices": [dict(name=m["name"], N=m["p"].N, K=m["p"].K) for m in mats],
            "weight_copies_rotated": [len(m["blobs"]) for m in mats],
        },
        "timing": "an untimed settle phase (the step repeated for settle_ms: the GPU's power management takes "
                  "20-40 ms of sustained load to settle), W untimed warm-up steps, then the K steps issued back "
                  "to back between one pair of events on the launch stream (each launch on its own weight copy, "
                  ">= 1 GiB rotated per matrix; each call's workspace allocated once before the timed region); "
                  "ms_per_step = the event pair's time / K; roofline.avg_launch_us = ms_per_step / the step's "
                  "launches; per_matrix.us: a second run of the same steps with an event before every launch "
                  "(event to next event; each event adds a gap of a few us, ms_per_step_events)",
        "settle_ms": SETTLE_MS,
        "dense_reference": "speedup_vs_dense: the same-shape dense GEMM = the same weights packed with every tile "
                           "dense, run by the same kernels (the sparsity gain alone); speedup_vs_rowmajor_dense: "
                           "patch_dense_gemm on row-major W; speedup_vs_hipblaslt: torch.matmul (hipBLASLt) against "
                           "the hybrid GEMM, both as 3 batches of K back-to-back launches between one event pair "
                           "(median; _events: the steps with an event before every launch)",
        "ms_per_step_graph": ms_step_graph,
        "ms_per_step_events": ms_step_ev,
        "speedup_vs_dense_step": ms_s0 / ms_step if refs else None,
        "speedup_vs_rowmajor_dense_step": ms_dense / ms_step if refs else None,
        "speedup_vs_hipblaslt_step": (sum(median(per_bb[m["name"]]) for m in mats) /
                                      sum(median(per_hb[m["name"]]) for m in mats)) if refs else None,
        "speedup_vs_hipblaslt_step_events": ms_blas_ev / ms_step_ev if refs else None,
        "per_matrix": per_matrix,
        "roofline": {
            "kernel": "prefill hybrid GEMM (packed W), both matrices' launches",
            "bound": "mfma",
            "achieved": achieved,
            "peak": MFMA_PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "flops_per_launch_effective": eff_sum / n_launch,
            "launches_per_step": n_launch,
            "avg_launch_us": avg_t * 1e6,
            "roofline_us_per_launch": tm_sum / n_launch * 1e6,
            "note": "achieved = effective flops (32768 a token a dense tile, 16384 a 2:4 tile) of a step / "
                    "ms_per_step; "
                    "effective work at the blended matrix-core peak (dense tiles at 2516.6, 2:4 tiles at twice "
                    "that, dense-equivalent) runs at exactly 2516.6 TFLOP/s, so frac = roofline time / time",
        },
    }
    return line, mats


def decode_extra(args):
    """The decode workload (LLaMA-2-7B q_proj 4096 x 4096, half the tiles
    2:4, M = 1, 4, 16): graph replays, each launch on its own weight copy."""
    import torch

    from sparse_gemm_amd import inputs, patch

    cfg = inputs.CONFIGS["decode"]
    Ms = cfg.Ms
    res = gemm_set("decode", 0, 0, Ms, args.steps, args.warmup, batches=3)
    p = res["p"]
    ns, T = int(p.tile_map.sum()), int(p.tile_map.size)
    summ = summarize(res, Ms)
    t_sum = sum(median(res["per"][M]) for M in Ms) * 1e-3
    b_sum = sum(algo_bytes(p.N, p.K, M, ns) for M in Ms)
    tr = [traffic_for("decode", M) for M in Ms]
    return {
        "workload": "decode: q_proj W 4096x4096 bf16, 512 of 1024 tiles 2:4 (25% sparsity), top-2-of-4 masks, "
                    "X M in {1,4,16}; one step = patch_gemm at each M, each launch on its own weight copy",
        "ms_per_step": res["ms_step"],
        "tflops_dense_equiv_step": sum(2.0 * M * p.N * p.K for M in Ms) / (res["ms_step"] * 1e-3) / 1e12,
        "sum_of_per_M_launches_ms": t_sum * 1e3,
        "speedup_vs_dense_step": res["ms_step_dense"] / res["ms_step"] if res["ms_step_dense"] else None,
        "speedup_vs_rowmajor_dense_step": (res["ms_step_rowmajor"] / res["ms_step"] if res["ms_step_rowmajor"]
                                           else None),
        "per_M": {str(M): summ[M] for M in Ms},
        "roofline": {"kernel": "decode hybrid GEMM", "bound": "hbm", "achieved": b_sum / t_sum / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": b_sum / t_sum / 1e9 / HBM_PEAK_GBS,
                     "traffic": (sum(tr) / len(tr)) if all(x is not None for x in tr) else None,
                     "bytes_per_launch_algorithmic": b_sum / len(Ms), "avg_launch_us": t_sum / len(Ms) * 1e6},
        "blob_bytes": res["pw"].nbytes,
        "weight_copies_rotated": res["n_copies"],
    }


def sweep_compact(steps, warmup, Ms=(1, 2048)):
    """The sparsity sweep on three LLaMA-2-7B shapes (q_proj, gate_proj,
    down_proj) at s = 0, .25, .5, .75, 1 and M in Ms: hybrid time, the
    same-shape dense kernel, and speedups; `monotone` says whether the
    speedup over the dense kernel rises strictly with s."""
    import torch

    from sparse_gemm_amd import inputs, patch

    cfg = inputs.CONFIGS["sweep"]
    out = []
    for mi in (0, 4, 6):
        p = inputs.make_weights(cfg, mi, 0)
        W = dev_bits(p.w, torch.bfloat16)
        mk = torch.from_numpy(p.mask).cuda()
        Ws = rotate(W, W.numel() * 2)
        Xs = {M: dev_bits(inputs.make_x(cfg, M, p.K, matrix_index=mi), torch.bfloat16) for M in Ms}
        Y = {M: torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for M in Ms}
        _, per_d = time_graphs([(M, (lambda i, M=M: patch.dense_gemm(Xs[M], Ws[i % len(Ws)], out=Y[M],
                                                                     workspace=ws_dense(M, p.N, p.K))))
                                for M in Ms], steps, warmup, 3)
        del Ws
        rec = {M: dict(matrix=cfg.matrices[mi].name, N=p.N, K=p.K, M=M, s=[], us=[],
                       rowmajor_dense_us=median(per_d[M]) * 1e3, roofline_frac=[]) for M in Ms}
        for si, frac in enumerate(cfg.fractions):
            q = inputs.make_weights(cfg, mi, si, reuse=p)
            pw = patch.pack(W, q.tile_map, mk)
            blobs = rotate(pw.blob, pw.nbytes)
            _, per = time_graphs([(M, (lambda i, M=M: patch.gemm(Xs[M], patch.PackedWeight(blobs[i % len(blobs)],
                                                                                            pw.desc), out=Y[M],
                                                                 workspace=ws_gemm(pw.desc, M))))
                                  for M in Ms], steps, warmup, 3)
            ns, T = int(q.tile_map.sum()), int(q.tile_map.size)
            for M in Ms:
                t = median(per[M]) * 1e-3
                r = rec[M]
                r["s"].append(ns / T)
                r["us"].append(t * 1e6)
                t_hbm = algo_bytes(p.N, p.K, M, ns) / (HBM_PEAK_GBS * 1e9)
                r["roofline_frac"].append(max(t_hbm, t_mfma_s(M, T, ns)) / t)
            del blobs, pw
            torch.cuda.empty_cache()
        for M in Ms:
            r = rec[M]
            # the dense reference: the s = 0 point (every tile dense, same kernels)
            r["speedup_vs_dense"] = [r["us"][0] / u for u in r["us"]]
            r["speedup_vs_rowmajor_dense"] = [r["rowmajor_dense_us"] / u for u in r["us"]]
            sp = r["speedup_vs_dense"]
            r["monotone"] = all(b > a for a, b in zip(sp, sp[1:]))
            out.append(r)
        del W, mk, Xs, Y
        torch.cuda.empty_cache()
    return out


def main():
    global HYBRID_ONLY, SETTLE_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline only (no decode workload, sweep or ceilings): for profiling")
    ap.add_argument("--report", default=None, help="also write the full sweep as JSON lines to this path")
    ap.add_argument("--report-steps", type=int, default=100, help="launches per timed batch in the report")
    ap.add_argument("--report-batches", type=int, default=10, help="timed batches per point in the report (median)")
    ap.add_argument("--workload", default="prefill_mlp",
                    choices=["prefill_mlp", "decode", "imbalanced_13b", "sampler", "fine_mask", "n48", "tile64"],
                    help="prefill_mlp (default: the headline line); the others print that workload's lines, "
                         "for profiling")
    ap.add_argument("--hybrid-only", action="store_true",
                    help="time the hybrid launches alone, no reference GEMMs (for profiler and counter runs, whose "
                         "per-kernel figures then cover the hybrid launches alone)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed settle phase before every timed measurement, ms (0: none)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for rocprofv3 byte counters)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR", default=None,
                    help="FETCH_DIR WRITE_DIR [FETCH_DIR WRITE_DIR ...]: write profiles/traffic_counters.json from "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE runs and exit")
    args = ap.parse_args()
    HYBRID_ONLY = args.hybrid_only
    SETTLE_MS = args.settle_ms
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 (the multi-GPU sharding "
                                   "is a design note, not a code path)"}))
        sys.exit(2)

    import torch

    from sparse_gemm_amd import inputs, patch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    patch.load()

    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel(), "copies": 3}), file=sys.stderr, flush=True)
        del src, dst
    if args.workload == "tile64":
        for rec in q64_set(args.steps, args.warmup):
            print(json.dumps(rec), flush=True)
        return
    if args.workload in ("sampler", "fine_mask", "n48"):
        fn = {"sampler": sampler_set, "fine_mask": fine_set, "n48": n48_set}[args.workload]
        for rec in fn(args.steps, args.warmup, 1):
            print(json.dumps(rec), flush=True)
        return
    if args.workload == "imbalanced_13b":
        run_prefill_workload(args)
        return
    if args.workload == "decode":
        print(json.dumps(decode_extra(args)), flush=True)
        return

    print("[bench] prefill MLP headline", file=sys.stderr, flush=True)
    line, mats = headline_prefill(args)
    problems = [(m["p"], inputs.CONFIGS["prefill_mlp"], i) for i, m in enumerate(mats)]
    Ms = [line["config"]["M"]] * len(mats)
    blob_sizes = [m["pw"].nbytes for m in mats]
    del mats
    torch.cuda.empty_cache()
    if not args.no_extras:
        print("[bench] decode workload", file=sys.stderr, flush=True)
        line["decode"] = decode_extra(args)
        print("[bench] ceilings", file=sys.stderr, flush=True)
        line["ceilings"] = measure_ceilings([line["decode"]["blob_bytes"], blob_sizes[0]])
        dec_b = str(line["decode"]["blob_bytes"] // 16 * 16)
        line["decode"]["roofline"]["measured_read_ceiling_gbps"] = line["ceilings"]["hbm_read"][dec_b]["gbps"]
        line["decode"]["roofline"]["frac_of_measured_ceiling"] = (line["decode"]["roofline"]["achieved"] /
                                                                  line["ceilings"]["hbm_read"][dec_b]["gbps"])
        sm = line["ceilings"]["matrix_core_tflops"]
        line["roofline"]["measured_ceilings_tflops"] = {k: sm[k] for k in sm}
        print("[bench] sparsity sweep", file=sys.stderr, flush=True)
        line["sweep"] = sweep_compact(max(10, args.steps), args.warmup)
        print("[bench] 64 x 64 execution tiles", file=sys.stderr, flush=True)
        line["tile64"] = q64_set(max(10, args.steps), args.warmup)
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(problems, Ms, sample_rows=32)
    print(json.dumps(line), flush=True)

    if args.report:
        write_report(args.report, args.report_steps, args.warmup, args.report_batches)


def run_prefill_workload(args):
    """One prefill workload (both matrices) as JSON lines: for profiling the
    prefill kernel; not the headline line."""
    from sparse_gemm_amd import inputs

    cfg = inputs.CONFIGS[args.workload]
    for mi in range(len(cfg.matrices)):
        res = gemm_set(args.workload, mi, 0, cfg.Ms, args.steps, args.warmup)
        summ = summarize(res, cfg.Ms)
        p = res["p"]
        for M in cfg.Ms:
            print(json.dumps(dict(workload=args.workload, matrix=cfg.matrices[mi].name, N=p.N, K=p.K, M=M,
                                  sparse_tiles=int(p.tile_map.sum()), tiles=int(p.tile_map.size),
                                  algorithmic_bytes=algo_bytes(p.N, p.K, M, int(p.tile_map.sum())),
                                  traffic_counters_bytes=traffic_for("prefill", M) if args.workload == "prefill_mlp"
                                  else None, **summ[M])),
                  flush=True)


def sampler_set(steps, warmup, batches):
    """The forward hybrid-mask sampler (patch_sample_mask) on the LLaMA-2-7B
    q_proj and gate_proj shapes, with and without the soft mask: graph
    replays of `steps` launches.  Inputs (float32 logits and uniforms, ~6 +
    6 bytes per weight) exceed the Infinity Cache on gate_proj and nearly on
    q_proj; HBM roofline on the algorithmic bytes: logits + uniforms read,
    tile map + mask (+ soft mask) written."""
    import torch

    from sparse_gemm_amd import inputs, patch

    out = []
    for name, N, K in (("q_proj", 4096, 4096), ("gate_proj", 11008, 4096)):
        s = inputs.make_sampler_inputs(N, K, 0, sparse_bias=0.4)
        dev = [torch.from_numpy(a).cuda() for a in (s.tile_logits, s.tile_u, s.pat_logits, s.pat_u)]
        bufs = (torch.empty((N // 128, K // 128), dtype=torch.uint8, device="cuda"),
                torch.empty((N, K), dtype=torch.uint8, device="cuda"),
                torch.empty((N, K), dtype=torch.float32, device="cuda"))
        T = (N // 128) * (K // 128)
        for soft in (True, False):
            fn = (lambda k, soft=soft: patch.sample_mask(*dev, 0.5, soft=soft, out=bufs))
            _, per = time_graphs([("s", fn)], steps, warmup, batches)
            us = median(per["s"]) * 1e3
            nbytes = N * (K // 4) * 6 * 4 * 2 + T * 2 * 4 * 2 + T + N * K + (4 * N * K if soft else 0)
            gbps = nbytes / (us * 1e-6) / 1e9
            out.append(dict(config="sampler", matrix=name, N=N, K=K, soft=soft, us=us, gbps=gbps,
                            algorithmic_bytes=nbytes, sparse_tile_fraction=float(bufs[0].float().mean().item()),
                            roofline_bound="hbm", roofline_frac=gbps / HBM_PEAK_GBS))
        del dev, bufs
        torch.cuda.empty_cache()
    return out


def n48_set(steps, warmup, batches, Ms=(1, 16, 128, 2048)):
    """4:8 tiles (the third tile kind) on the LLaMA-2-7B q_proj, gate_proj
    and down_proj shapes: every tile 4:8, every tile 2:4 and every tile
    dense (the dense kernel on row-major W), top-4-of-8 / top-2-of-4
    masks; graph replays, rotated copies as elsewhere."""
    import torch

    from sparse_gemm_amd import inputs, patch

    out = []
    for name, N, K in (("q_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("down_proj", 4096, 11008)):
        p48 = inputs.make_mixed("bf16", N, K, 0, 0.0, 1.0)
        p24 = inputs.make_mixed("bf16", N, K, 0, 1.0, 0.0)
        W = dev_bits(p48.w, torch.bfloat16)
        packs = {}
        for tag, p in (("48", p48), ("24", p24)):
            pw = patch.pack(W, p.tile_map, torch.from_numpy(p.mask).cuda())
            packs[tag] = (rotate(pw.blob, pw.nbytes), pw.desc)
        Ws = rotate(W, W.numel() * 2)
        for M in Ms:
            X = dev_bits(inputs.make_x(inputs.CONFIGS["sweep"], M, K), torch.bfloat16)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            calls = [(tag, (lambda k, b=b, d=d, M=M: patch.gemm(X, patch.PackedWeight(b[k % len(b)], d), out=Y,
                                                                workspace=ws_gemm(d, M))))
                     for tag, (b, d) in packs.items()]
            calls.append(("dense", lambda k, M=M: patch.dense_gemm(X, Ws[k % len(Ws)], out=Y,
                                                                   workspace=ws_dense(M, N, K))))
            _, per = time_graphs(calls, steps, warmup, batches)
            us = {t: median(v) * 1e3 for t, v in per.items()}
            out.append(dict(config="n48", matrix=name, N=N, K=K, M=M, us_48=us["48"], us_24=us["24"],
                            us_dense=us["dense"], speedup_48_vs_dense=us["dense"] / us["48"],
                            speedup_24_vs_dense=us["dense"] / us["24"],
                            tflops_dense_equiv_48=2.0 * M * N * K / (us["48"] * 1e-6) / 1e12,
                            gbps_48=algo_bytes(N, K, M, (N // 128) * (K // 128)) / (us["48"] * 1e-6) / 1e9))
        del packs, Ws, W
        torch.cuda.empty_cache()
    return out


def q64_set(steps, warmup, batches=3):
    """64 x 64 against 128 x 128 execution tiles for one mask learnt on
    64 x 64 tiles (LLaMA-2-7B q_proj 4096 x 4096 and gate_proj 11008 x 4096,
    bf16; a 128 x 128 tile is 2:4 in all four quadrants with probability 0.4,
    else each quadrant is 2:4 with probability 0.6; uniformly drawn 2:4
    patterns), at M = 1, 16 and 2048, each launch on its own weight copy,
    graph replays (median of batches):
      * q64: the 64 x 64 blob (patch_pack_q64), every 2:4 quadrant on the
        sparse path;
      * t128: the 128 x 128 blob under the all-2:4 policy (a tile runs 2:4
        only if its four quadrants are; dense tiles on W o E_fine:
        patch_exec_tile_map + patch_apply_fine_mask + patch_pack) -- the same
        product X (W o E_fine)^T;
      * dense: the same weights packed with every tile dense (same kernels)."""
    import torch

    from sparse_gemm_amd import inputs, patch

    out = []
    for name, N, K in (("q_proj", 4096, 4096), ("gate_proj", 11008, 4096)):
        p = inputs.make_fine("bf16", N, K, 64, 64, 0)
        W = dev_bits(p.w, torch.bfloat16)
        mk = torch.from_numpy(p.mask).cuda()
        packs = {"q64": patch.pack_q64(W, p.tile_map, mk), "t128": patch.pack_fine(W, p.tile_map, mk, 64, 64),
                 "dense": patch.pack(W, np.zeros((N // 128, K // 128), np.uint8), mk)}
        del mk
        emap = patch.exec_tile_map(N, K, p.tile_map, 64, 64)
        rec = dict(config="tile64", matrix=name, N=N, K=K, quadrant_sparse_fraction=float(p.tile_map.mean()),
                   tile128_sparse_fraction=float(emap.mean()),
                   blob_bytes={k: v.nbytes for k, v in packs.items()}, us={})
        Ms = (1, 16, 2048)
        Xs = {M: dev_bits(inputs.make_x(inputs.CONFIGS["decode"], M, K), torch.bfloat16) for M in Ms}
        Ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M in Ms}
        for k, pw in packs.items():
            blobs = rotate(pw.blob, pw.nbytes)

            def mk_fn(M, blobs=blobs, desc=pw.desc):
                return lambda i: patch.gemm(Xs[M], patch.PackedWeight(blobs[i % len(blobs)], desc), out=Ys[M],
                                            workspace=ws_gemm(desc, M))

            _, per = time_graphs([(M, mk_fn(M)) for M in Ms], steps, warmup, batches)
            rec["us"][k] = {str(M): median(per[M]) * 1e3 for M in Ms}
            del blobs
            torch.cuda.empty_cache()
        rec["speedup_q64_vs_t128"] = {str(M): rec["us"]["t128"][str(M)] / rec["us"]["q64"][str(M)] for M in Ms}
        rec["speedup_q64_vs_dense"] = {str(M): rec["us"]["dense"][str(M)] / rec["us"]["q64"][str(M)] for M in Ms}
        rec["speedup_t128_vs_dense"] = {str(M): rec["us"]["dense"][str(M)] / rec["us"]["t128"][str(M)] for M in Ms}
        out.append(rec)
        del W, packs, Xs, Ys
        torch.cuda.empty_cache()
    return out


def fine_set(steps, warmup, batches):
    """patch_apply_fine_mask (W o E_fine for the dense execution tiles of a
    mask learnt on finer tiles) on the LLaMA-2-7B gate_proj shape with 32 x 32
    and 4 x 4 mask tiles: graph replays; HBM roofline on W read (2 B), mask
    read (1 B) and W_out written (2 B) per weight."""
    import torch

    from sparse_gemm_amd import inputs, patch

    out = []
    N, K = 11008, 4096
    for b1, b2 in ((32, 32), (4, 4)):
        p = inputs.make_fine("bf16", N, K, b1, b2, 0)
        W = torch.from_numpy(p.w.view(np.int16)).view(torch.bfloat16).cuda()
        fm = torch.from_numpy(p.tile_map).cuda()
        mk = torch.from_numpy(p.mask).cuda()
        Wo = torch.empty_like(W)
        fn = (lambda k: patch.apply_fine_mask(W, fm, mk, b1, b2, out=Wo))
        _, per = time_graphs([("f", fn)], steps, warmup, batches)
        us = median(per["f"]) * 1e3
        nbytes = 5 * N * K + p.tile_map.size
        gbps = nbytes / (us * 1e-6) / 1e9
        emap = patch.exec_tile_map(N, K, p.tile_map, b1, b2)
        out.append(dict(config="fine_mask", matrix="gate_proj", N=N, K=K, b1=b1, b2=b2, us=us, gbps=gbps,
                        algorithmic_bytes=nbytes, fine_sparse_fraction=float(p.tile_map.mean()),
                        exec_sparse_fraction=float(emap.mean()), roofline_bound="hbm",
                        roofline_frac=gbps / HBM_PEAK_GBS))
        del W, fm, mk, Wo
        torch.cuda.empty_cache()
    return out


def fused_set(kind, si, Ms, steps, warmup, batches):
    """Fused projections of the sweep's LLaMA-2-7B weights at sparse-tile
    fraction index si, one record per M:
      kind "swiglu": gate_proj + up_proj -> H = SiLU(X Wg^T) * (X Wu^T):
        fused (patch_gemm_swiglu, one launch) against the two hybrid GEMMs plus
        torch's elementwise SiLU * mul, the same-shape dense fused kernel
        (patch_dense_gemm_swiglu) and hipBLASLt (two torch.matmul + SiLU * mul,
        eager);
      kind "qkv": q_proj, k_proj, v_proj packed as one blob: one patch_gemm
        against three, the dense kernel on the concatenated weight and
        hipBLASLt (three torch.matmul, eager).
    Our kernels are timed as graph replays (as elsewhere), hipBLASLt eagerly."""
    import torch

    from sparse_gemm_amd import inputs, patch

    cfg = inputs.CONFIGS["sweep"]
    mis = (4, 5) if kind == "swiglu" else (0, 1, 2)
    ps = [inputs.make_weights(cfg, mi, si) for mi in mis]
    tdt = torch.bfloat16
    Ws = [dev_bits(p.w, tdt) for p in ps]
    masks = [torch.from_numpy(p.mask).cuda() for p in ps]
    singles = [patch.pack(W, p.tile_map, mk) for W, p, mk in zip(Ws, ps, masks)]
    if kind == "swiglu":
        fused = patch.pack_gate_up(Ws[0], Ws[1], ps[0].tile_map, ps[1].tile_map, masks[0], masks[1])
    else:
        fused = patch.pack_concat(Ws, [p.tile_map for p in ps], masks)
    del masks
    K = ps[0].K
    Ntot = sum(p.N for p in ps)
    F = ps[0].N
    blobs = rotate(fused.blob, fused.nbytes)
    sblobs = [rotate(sp.blob, sp.nbytes) for sp in singles]
    Wcat = torch.cat(Ws) if kind == "qkv" else None
    Wrot = rotate(Wcat, Wcat.numel() * 2) if kind == "qkv" else None
    Wg_rot = rotate(Ws[0], Ws[0].numel() * 2) if kind == "swiglu" else None
    Wu_rot = rotate(Ws[1], Ws[1].numel() * 2) if kind == "swiglu" else None
    out = {}
    for M in Ms:
        X = dev_bits(inputs.make_x(cfg, M, K, matrix_index=mis[0]), tdt)
        outw = F if kind == "swiglu" else Ntot
        Y = torch.empty((M, outw), dtype=tdt, device="cuda")
        Ys = [torch.empty((M, p.N), dtype=tdt, device="cuda") for p in ps]

        if kind == "swiglu":
            def f_fused(k):
                patch.gemm_swiglu(X, patch.PackedWeight(blobs[k % len(blobs)], fused.desc), out=Y,
                                  workspace=ws_swiglu(fused.desc, M))

            def f_unfused(k):
                for sb, sp, y in zip(sblobs, singles, Ys):
                    patch.gemm(X, patch.PackedWeight(sb[k % len(sb)], sp.desc), out=y, workspace=ws_gemm(sp.desc, M))
                torch.mul(torch.nn.functional.silu(Ys[0]), Ys[1], out=Y)

            def f_dense(k):
                patch.dense_gemm_swiglu(X, Wg_rot[k % len(Wg_rot)], Wu_rot[k % len(Wu_rot)], out=Y)

            def f_blas(k):
                torch.matmul(X, Wg_rot[k % len(Wg_rot)].t(), out=Ys[0])
                torch.matmul(X, Wu_rot[k % len(Wu_rot)].t(), out=Ys[1])
                torch.mul(torch.nn.functional.silu(Ys[0]), Ys[1], out=Y)
        else:
            def f_fused(k):
                patch.gemm(X, patch.PackedWeight(blobs[k % len(blobs)], fused.desc), out=Y,
                           workspace=ws_gemm(fused.desc, M))

            def f_unfused(k):
                for sb, sp, y in zip(sblobs, singles, Ys):
                    patch.gemm(X, patch.PackedWeight(sb[k % len(sb)], sp.desc), out=y, workspace=ws_gemm(sp.desc, M))

            def f_dense(k):
                patch.dense_gemm(X, Wrot[k % len(Wrot)], out=Y, workspace=ws_dense(M, Ntot, K))

            def f_blas(k):
                Wr = Wrot[k % len(Wrot)]
                for i, y in enumerate(Ys):
                    torch.matmul(X, Wr[4096 * i:4096 * (i + 1)].t(), out=y)

        _, per_g = time_graphs([("fused", f_fused), ("unfused", f_unfused), ("dense", f_dense)], steps, warmup,
                               batches)
        _, per_e = time_launches([("fused", f_fused), ("unfused", f_unfused), ("blas", f_blas)], steps, warmup,
                                 batches)
        t = median(per_g["fused"]) * 1e-3
        ns = sum(int(p.tile_map.sum()) for p in ps)
        T = sum(int(p.tile_map.size) for p in ps)
        nbytes = 256 + 16 * T + 32768 * (T - ns) + 18432 * ns + 2 * M * K + 2 * M * outw
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mma = 2.0 * M * 128 * 128 * ((T - ns) / MFMA_PEAK_BF16_TFLOPS + ns / (2 * MFMA_PEAK_BF16_TFLOPS)) / 1e12
        out[M] = dict(us=t * 1e6, us_unfused=median(per_g["unfused"]) * 1e3, us_dense=median(per_g["dense"]) * 1e3,
                      us_eager=median(per_e["fused"]) * 1e3, us_unfused_eager=median(per_e["unfused"]) * 1e3,
                      hipblaslt_us_eager=median(per_e["blas"]) * 1e3,
                      speedup_vs_unfused=median(per_g["unfused"]) * 1e-3 / t,
                      speedup_vs_dense=median(per_g["dense"]) * 1e-3 / t,
                      speedup_vs_hipblaslt_eager=median(per_e["blas"]) / median(per_e["fused"]),
                      tflops_dense_equiv=2.0 * M * Ntot * K / t / 1e12, gbps=nbytes / t / 1e9,
                      roofline_bound="hbm" if t_hbm >= t_mma else "mfma", roofline_frac=max(t_hbm, t_mma) / t,
                      N_total=Ntot, K=K, sparse_tile_fraction=ns / T)
    del blobs, sblobs, Wrot, Wg_rot, Wu_rot
    torch.cuda.empty_cache()
    return out


def write_report(path, steps, warmup, batches):
    """Every workload: decode, prefill MLP, the sparsity sweep and the 13B
    imbalanced shapes; one JSON line per (matrix, s, M).  Each time is the
    median of `batches` batches of `steps` launches (min and max beside it)."""
    from sparse_gemm_amd import inputs

    with open(path, "w") as f:
        def emit(cfg_name, mi, si, Ms, fraction=None, map_kind=None):
            cfg = inputs.CONFIGS[cfg_name]
            res = gemm_set(cfg_name, mi, si, Ms, steps, warmup, fraction=fraction, map_kind=map_kind,
                           batches=batches)
            summ = summarize(res, Ms)
            p = res["p"]
            for M in Ms:
                rec = dict(config=cfg_name, matrix=cfg.matrices[mi].name, N=p.N, K=p.K, M=M,
                           sparse_tile_fraction=float(p.tile_map.mean()), sparse_tiles=int(p.tile_map.sum()),
                           pack_us=res["pack_ms"] * 1e3, **summ[M])
                f.write(json.dumps(rec) + "\n")
                f.flush()
                print(f"[report] {cfg_name} {rec['matrix']} s={rec['sparse_tile_fraction']:.3f} M={M}: "
                      f"{rec['us']:.2f} us, {rec['tflops_dense_equiv']:.1f} TFLOP/s, x{rec['speedup_vs_dense']:.3f} "
                      f"vs dense, roofline {rec['roofline_frac']:.2f}", flush=True)

        emit("tiny", 0, 0, (16,))
        emit("decode", 0, 0, (1, 4, 16))
        for mi in range(2):
            emit("prefill_mlp", mi, 0, (2048,))
        for mi in range(2):
            emit("imbalanced_13b", mi, 0, (4096,))
        for mi in (0, 4, 6):  # q_proj-like, gate/up-like, down
            for si in range(5):
                emit("sweep", mi, si, (1, 16, 128, 2048))
        for rec in n48_set(steps, warmup, batches):
            f.write(json.dumps(rec) + "\n")
            f.flush()
            print(f"[report] 4:8 {rec['matrix']} M={rec['M']}: {rec['us_48']:.2f} us (2:4 {rec['us_24']:.2f}, dense "
                  f"{rec['us_dense']:.2f}), x{rec['speedup_48_vs_dense']:.3f} vs dense", flush=True)
        for rec in fine_set(steps, warmup, batches):
            f.write(json.dumps(rec) + "\n")
            f.flush()
            print(f"[report] fine mask {rec['b1']}x{rec['b2']}: {rec['us']:.2f} us, {rec['gbps']:.0f} GB/s, "
                  f"roofline {rec['roofline_frac']:.2f}", flush=True)
        for rec in sampler_set(steps, warmup, batches):
            f.write(json.dumps(rec) + "\n")
            f.flush()
            print(f"[report] sampler {rec['matrix']} soft={rec['soft']}: {rec['us']:.2f} us, {rec['gbps']:.0f} GB/s, "
                  f"roofline {rec['roofline_frac']:.2f}", flush=True)
        for kind in ("swiglu", "qkv"):
            for si in (0, 2, 4):
                res = fused_set(kind, si, (1, 16, 128, 2048), steps, warmup, batches)
                for M, rec in res.items():
                    rec = dict(config="fused_" + kind, matrix=kind, M=M, **rec)
                    f.write(json.dumps(rec) + "\n")
                    f.flush()
                    print(f"[report] fused {kind} s={rec['sparse_tile_fraction']:.2f} M={M}: {rec['us']:.2f} us, "
                          f"x{rec['speedup_vs_unfused']:.3f} vs unfused, x{rec['speedup_vs_dense']:.3f} vs dense",
                          flush=True)


if __name__ == "__main__":
    main()
