#!/usr/bin/env python3
"""Throughput of the PATCH hybrid tile-sparse GEMM on one MI355X.

PATCH (arXiv 2509.23410): every 128 x 128 tile of W is dense or 2:4 sparse
(gist.science explainer, section 2 "Core Mechanism"); the pages report only
end-to-end numbers (1.18x-1.38x over dense, LLaMA-2 7B on an A6000, section 4
"Speedup & Efficiency"), so there is no published kernel figure to compare
with and vs_baseline is null.

Default workload: the LLaMA-2-7B q_proj decode GEMM -- W 4096 x 4096 bf16,
half of the 1024 tiles 2:4 (25% sparsity), top-2-of-4 masks, X with
M = 1, 4 and 16 rows.  One step = one patch_gemm call for each M (every
kernel of the hot path at inference: the decode hybrid GEMM with its
epilogue; packing is offline and timed separately).  Inputs are resident in
HBM; 40 copies of the packed weight are rotated so the 256 MB Infinity Cache
cannot serve them.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--report out.jsonl]

Prints one JSON line.  --report also writes the sweep over all workloads
(every sparse-tile fraction, decode and prefill shapes) as JSON lines.
"""
from __future__ import annotations

import argparse
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
KERNEL_SOURCES = ("sparse_gemm_amd/csrc/gemm_decode.hip", "sparse_gemm_amd/csrc/gemm_prefill.hip",
                  "sparse_gemm_amd/csrc/device_common.h")


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


def time_launches(calls, steps, warmup, batches=1):
    """calls: list of (key, fn(k)).  Returns
      * ms per step, a step running every call once, back to back (one event
        pair around all `steps` steps), and
      * {key: [ms per launch of each batch]}, each call timed on its own:
        `batches` batches of `steps` launches back to back, one event pair
        around each batch, divided by `steps`.
    Events are recorded on the current stream, the one the launches use."""
    import torch

    for k in range(warmup):
        for _, fn in calls:
            fn(k)
    torch.cuda.synchronize()
    a = _event()
    for k in range(steps):
        for _, fn in calls:
            fn(warmup + k)
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
    """As time_launches, but the launches are captured in HIP graphs and the
    graphs replayed, so host launch overhead is out of the timed region:
      * ms per step: one graph of `steps` steps (every call once a step, back
        to back), replayed once untimed and once between one event pair;
      * {key: [ms per launch of each batch]}: per call, one graph of `steps`
        launches, replayed `batches` times, each between one event pair.
    Step k of either uses rotation index warmup + k, as the eager timing."""
    import torch

    for k in range(warmup):
        for _, fn in calls:
            fn(k)
    torch.cuda.synchronize()
    g = _capture([(lambda fn=fn, k=k: fn(warmup + k)) for k in range(steps) for _, fn in calls])
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
    import torch

    n = max(2, min(64, int(np.ceil(ROTATE_BYTES / max(1, nbytes_each)))))
    return [t] + [t.clone() for _ in range(n - 1)]


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
    del mask
    blobs = rotate(pw.blob, pw.nbytes)
    Ws = rotate(W, W.numel() * 2)
    Xs = {M: dev_bits(inputs.make_x(cfg, M, p.K, matrix_index=mi), tdt) for M in Ms}
    Ys = {M: torch.empty((M, p.N), dtype=tdt, device="cuda") for M in Ms}
    desc = pw.desc

    def hyb(M):
        def f(k):
            patch.gemm(Xs[M], patch.PackedWeight(blobs[k % len(blobs)], desc), out=Ys[M])
        return f

    def dense(M):
        def f(k):
            patch.dense_gemm(Xs[M], Ws[k % len(Ws)], out=Ys[M])
        return f

    def blas(M):
        def f(k):
            torch.matmul(Xs[M], Ws[k % len(Ws)].t(), out=Ys[M])
        return f

    # our kernels: graph replays (launch overhead out of the timed region)
    # and eager back-to-back launches; hipBLASLt (torch.matmul): eager only,
    # since a library call may record work that graph replays do not repeat
    # faithfully
    ms_h, per_h = time_graphs([(M, hyb(M)) for M in Ms], steps, warmup, batches)
    ms_d, per_d = time_graphs([(M, dense(M)) for M in Ms], steps, warmup, batches)
    ms_he, per_he = time_launches([(M, hyb(M)) for M in Ms], steps, warmup, batches)
    per_b = None
    if with_hipblaslt:
        _, per_b = time_launches([(M, blas(M)) for M in Ms], steps, warmup, batches)
    res = dict(p=p, pw=pw, pack_ms=pack_ms, ms_step=ms_h, ms_step_dense=ms_d, per=per_h, per_dense=per_d,
               ms_step_eager=ms_he, per_eager=per_he, per_blas=per_b, n_copies=len(blobs))
    del blobs, Ws
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
        td = median(res["per_dense"][M]) * 1e-3
        fl = 2.0 * M * N * K
        eff = 2.0 * M * N * K * (1 - 0.5 * s)
        e = dict(us=t * 1e6, us_min=min(res["per"][M]) * 1e3, us_max=max(res["per"][M]) * 1e3,
                 batches=len(res["per"][M]), us_eager=median(res["per_eager"][M]) * 1e3, dense_us=td * 1e6, tflops_dense_equiv=fl / t / 1e12, tflops_effective=eff / t / 1e12,
                 gbps=algo_bytes(N, K, M, ns) / t / 1e9, speedup_vs_dense=td / t)
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


def cpu_baseline(p, Ms, cfg):
    """The oracle, as it stands, on a bounded sample of the same step."""
    import oracle
    from sparse_gemm_amd import inputs

    Xb = {M: inputs.make_x(cfg, M, p.K) for M in Ms}
    flops = sum(2.0 * M * p.N * p.K for M in Ms)
    reps, t0 = 0, time.perf_counter()
    while True:
        for M in Ms:
            oracle.gemm_f64(p.dtype, Xb[M], p.w, p.tile_map, p.mask)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 5000:
            break
    return dict(value=flops * reps / el / 1e12, unit="TFLOP/s (dense-equivalent)", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"{reps} full step(s): oracle_gemm_f64 (fp64) for M in {list(Ms)} on the same "
                       f"{p.N}x{p.K} weights, tile map and masks; {el:.1f} s wall")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--report", default=None, help="also write the full sweep as JSON lines to this path")
    ap.add_argument("--report-steps", type=int, default=100, help="launches per timed batch in the report")
    ap.add_argument("--report-batches", type=int, default=10, help="timed batches per point in the report (median)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill_mlp", "imbalanced_13b", "sampler", "fine_mask", "n48"],
                    help="decode (default: the q_proj decode GEMM), a prefill workload or the mask sampler, "
                         "for profiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for rocprofv3 byte counters)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR", default=None,
                    help="FETCH_DIR WRITE_DIR [FETCH_DIR WRITE_DIR ...]: write profiles/traffic_counters.json from "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE runs and exit")
    args = ap.parse_args()
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
    if args.workload in ("sampler", "fine_mask", "n48"):
        fn = {"sampler": sampler_set, "fine_mask": fine_set, "n48": n48_set}[args.workload]
        for rec in fn(args.steps, args.warmup, 1):
            print(json.dumps(rec), flush=True)
        return
    if args.workload != "decode":
        run_prefill_workload(args)
        return
    cfg = inputs.CONFIGS["decode"]
    Ms = cfg.Ms
    res = gemm_set("decode", 0, 0, Ms, args.steps, args.warmup)
    p = res["p"]
    ns = int(p.tile_map.sum())
    summ = summarize(res, Ms)
    flops_step = sum(2.0 * M * p.N * p.K for M in Ms)
    value = flops_step / (res["ms_step"] * 1e-3) / 1e12

    # dominant kernel: the decode hybrid GEMM (all three launches of a step)
    t_sum = sum(mean(res["per"][M]) for M in Ms) * 1e-3
    b_sum = sum(algo_bytes(p.N, p.K, M, ns) for M in Ms)
    achieved = b_sum / t_sum / 1e9
    traffic = None
    tr = [traffic_for("decode", M) for M in Ms]
    if all(x is not None for x in tr):
        traffic = sum(tr) / len(tr)
    line = {
        "metric": "hybrid GEMM TFLOP/s (dense-equiv) + speedup vs dense, LLaMA-2-7B shapes",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) X, N(0,0.02) W; LLaMA-2-7B q_proj shape, no weights)",
        "config": {
            "workload": "decode: q_proj W 4096x4096 bf16, 512 of 1024 128x128 tiles 2:4 (25% sparsity), "
                        "top-2-of-4 masks, X M in {1,4,16}; one step = patch_gemm at each M",
            "N": p.N, "K": p.K, "Ms": list(Ms), "sparse_tiles": ns, "tiles": int(p.tile_map.size),
            "weight_copies_rotated": res["n_copies"],
        },
        "ms_per_step_eager": res["ms_step_eager"],
        "timing": "value and ms_per_step: one HIP graph of the K steps (3 patch_gemm launches each, cycling the "
                  "weight copies), replayed between one event pair; ms_per_step_eager: the same launches issued "
                  "from Python back to back",
        "speedup_vs_dense_step": res["ms_step_dense"] / res["ms_step"],
        "per_M": {str(M): summ[M] for M in Ms},
        "pack": {"us": res["pack_ms"] * 1e3,
                 "gbps": (2 * p.N * p.K + p.N * p.K + res["pw"].nbytes) / (res["pack_ms"] * 1e-3) / 1e9,
                 "note": "patch_pack incl. host header upload and stream sync; bytes = W + mask + blob"},
        "roofline": {
            "kernel": "k_decode (hybrid, packed W)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "bytes_per_launch_algorithmic": b_sum / len(Ms),
            "avg_launch_us": t_sum / len(Ms) * 1e6,
        },
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(p, Ms, cfg)
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
            calls = [(tag, (lambda k, b=b, d=d: patch.gemm(X, patch.PackedWeight(b[k % len(b)], d), out=Y)))
                     for tag, (b, d) in packs.items()]
            calls.append(("dense", lambda k: patch.dense_gemm(X, Ws[k % len(Ws)], out=Y)))
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
                patch.gemm_swiglu(X, patch.PackedWeight(blobs[k % len(blobs)], fused.desc), out=Y)

            def f_unfused(k):
                for sb, sp, y in zip(sblobs, singles, Ys):
                    patch.gemm(X, patch.PackedWeight(sb[k % len(sb)], sp.desc), out=y)
                torch.mul(torch.nn.functional.silu(Ys[0]), Ys[1], out=Y)

            def f_dense(k):
                patch.dense_gemm_swiglu(X, Wg_rot[k % len(Wg_rot)], Wu_rot[k % len(Wu_rot)], out=Y)

            def f_blas(k):
                torch.matmul(X, Wg_rot[k % len(Wg_rot)].t(), out=Ys[0])
                torch.matmul(X, Wu_rot[k % len(Wu_rot)].t(), out=Ys[1])
                torch.mul(torch.nn.functional.silu(Ys[0]), Ys[1], out=Y)
        else:
            def f_fused(k):
                patch.gemm(X, patch.PackedWeight(blobs[k % len(blobs)], fused.desc), out=Y)

            def f_unfused(k):
                for sb, sp, y in zip(sblobs, singles, Ys):
                    patch.gemm(X, patch.PackedWeight(sb[k % len(sb)], sp.desc), out=y)

            def f_dense(k):
                patch.dense_gemm(X, Wrot[k % len(Wrot)], out=Y)

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
