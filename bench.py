"""Throughput of the HIP verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one spec_verify_run (rows kernel + draw kernel) over the workload
B=64, gamma=5, V=151936, bf16 target logits, fp32 draft probabilities,
T=0.8 on every request.  Inputs are synthetic (seeded, see synth/), already
resident in HBM; R rotating copies of the inputs (more than the 256 MB
Infinity Cache can hold) are cycled so every step streams from HBM.

Before any GPU call the CPU oracle is timed on the same workload, in one
process and in a pool of forked workers over request chunks (the host's cores,
at most 16).  Then: the timed region (exactly K steps between two
synchronisations), a pass with an event between consecutive steps for the
median / p10 / p90 step time, a pass whose kernels are stamped by their own
dispatches (kernel durations without the gap between dispatches, as rocprofv3
reports them), and a plain streaming read of 1 GiB and of one step's bytes for
the device's practical read ceiling.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "spec-verify steps/s + HBM GB/s (% of peak) at B=64, γ=5, V=151936"
PEAK_HBM_GBPS = 8000.0
CONFIG_ID = 3
KDT = "BF16"
CSRC = os.path.join(ROOT, "lossless_rejection_sampling_sampler_amd", "csrc")
KERNEL_SOURCES = ("sv_device.h", "spec_verify.hip")


def _sparse_as_dense(rep):
    """The sparse workload's q kept in dense rows (the same q; for comparison)."""
    from synth.workloads import CONFIGS, make_inputs
    spec = CONFIGS[5].with_(q_mode="topk", name="B256_ragged8_V128256_bf16_top50_dense")
    return make_inputs(spec, seed=5100 + rep)


def make_workload(name: str, rep: int):
    from synth import make_config, make_point_config, make_sparse_config
    if name == "config3":
        return make_config(CONFIG_ID, replicate=rep)
    if name in ("config1", "config2", "config4", "config5"):
        return make_config(int(name[-1]), replicate=rep)
    if name == "sparse":
        return make_sparse_config(replicate=rep)
    if name == "sparse_as_dense":
        return _sparse_as_dense(rep)
    if name == "point":
        return make_point_config(replicate=rep)
    if name == "shard4":
        return make_config(CONFIG_ID, replicate=rep, vocab=151936 // 4, name="B64_g5_V37984_bf16_shard")
    if name == "sample":
        from synth import make_sample_config
        return make_sample_config(replicate=rep)
    if name == "point_as_dense":
        from synth.workloads import CONFIGS, make_inputs
        return make_inputs(CONFIGS[3].with_(q_mode="argmax", name="B64_g5_V151936_bf16_argmax_dense"),
                           seed=3100 + rep)
    raise ValueError(name)


GRAPH_CALLS = 16           # calls per captured graph in the multi-call graph timing


WORKLOAD_TEXT = {
    "config3": "B=64, gamma=5, V=151936, bf16 logits, fp32 q, T=0.8",
    "config1": "B=1, gamma=4, V=1000, fp32 logits, fp32 q, T=1",
    "config2": "B=8, gamma=5, V=32000, fp32 logits, fp32 q, T=1",
    "config4": "B=128, gamma=8, V=151936, bf16 logits, fp32 q, T mix {0, 0.3, 0.7, 1}",
    "config5": "B=256, ragged gamma_b in 0..8, V=128256, bf16 logits, half q = p, half top-50 dense q, T=1",
    "sparse": "B=256, ragged gamma_b in 0..8, V=128256, bf16 logits, top-50 q as 50 (id, prob) entries per row, T=1",
    "sparse_as_dense": "B=256, ragged gamma_b in 0..8, V=128256, bf16 logits, top-50 q in dense fp32 rows, T=1",
    "point": "B=64, gamma=5, V=151936, bf16 logits, point-mass drafts (no q memory), T=0.8",
    "point_as_dense": "B=64, gamma=5, V=151936, bf16 logits, point-mass drafts as one-hot dense fp32 q rows, T=0.8",
    "sample": "draft-side sampling: B=64 rows, gamma=0, V=151936, bf16 logits, T=0.8",
    "shard4": "one vocabulary shard of four: B=64, gamma=5, V=37984, bf16 logits, fp32 q, T=0.8",
}


def traffic_path(kernel: str) -> str:
    """Counter-derived HBM traffic of one kernel on this workload (written from rocprofv3 runs)."""
    stem = kernel.replace("<", "_").replace(">", "")
    return os.path.join(ROOT, "profiles", f"{stem}_B64_g5_V151936_traffic.json")


def kernel_source_sha() -> str:
    """Hash of the kernel sources with comments and blank lines dropped (a change
    of wording does not void a counter record; any change of code does)."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        for line in open(os.path.join(CSRC, f), encoding="utf-8"):
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(inp, num_accepted):
    """Bytes the method must move for one step (bytes it avoids are not counted).

    rows kernel: every target row once, the drafted-token gathers (id, logit and
    q: one value of a dense q row, the K (id, prob) entries of a sparse row, none
    for a point mass), temperature, uniforms and the outputs; draw kernel: the
    draw row's logits again for every sampled request and, for a residual, its
    q (a dense q row, or the sparse entries and their tokens' logits, or the
    drafted token and its logit for a point mass).
    """
    import numpy as np
    B, G, V, D, R = inp.batch, inp.gamma, inp.vocab, inp.total_draft, inp.total_rows
    sl = 2 if inp.dtype == "bf16" else 4
    sampled = inp.temperature > 0
    gam = inp.gammas
    fmt = getattr(inp, "q_format", "dense")
    K = inp.topk_ids.shape[1] if fmt == "sparse" else 0
    q_gather = {"dense": 4, "sparse": 8 * K, "point": 0}[fmt]
    q_residual = {"dense": 4 * V, "sparse": K * (8 + sl), "point": 4 + sl}[fmt]
    rows = R * V * sl + D * (4 + sl + q_gather) + 4 * B + 4 * B * (G + 2) + 4 * B * (G + 1) + 4 * B
    if inp.offsets is not None:
        rows += 4 * (B + 1)
    residual = sampled & (num_accepted < gam)
    draw = int(sampled.sum()) * V * sl + int(residual.sum()) * q_residual
    return int(rows), int(draw)


def traffic_entry(kernel: str):
    """HBM bytes per launch of ``kernel`` from rocprofv3 counters, or None when the
    record is missing or was taken from other kernel sources."""
    try:
        rec = json.load(open(traffic_path(kernel)))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30         # counter scale reference: bytes read (and written) per copy
COPY_REPS = 3


def read_counters(path):
    """{kernel name: (dispatches, mean counter value per dispatch)} of one rocprofv3
    counter_collection.csv (values of one dispatch summed over its rows)."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        n, tot = out.get(name, (0, 0.0))
        out[name] = (n + 1, tot + v)
    return {k: (n, tot / n) for k, (n, tot) in out.items()}


def write_traffic(fetch_csv, write_csv):
    """Counter-derived HBM bytes per launch of every verify kernel.  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are each scaled by what the same counter reads for
    the elementwise copy of COPY_BYTES (so the figure is in the copy's terms)."""
    fetch, write = read_counters(fetch_csv), read_counters(write_csv)
    copy = [k for k in fetch if "elementwise" in k and fetch[k][0] >= COPY_REPS]
    if not copy:
        raise SystemExit("no elementwise copy kernel in the counter file")
    ck = max(copy, key=lambda k: fetch[k][1])
    f_scale = COPY_BYTES / (fetch[ck][1] * 1024.0)
    w_scale = COPY_BYTES / (write[ck][1] * 1024.0)
    sha = kernel_source_sha()
    for name in fetch:
        short = None
        for kn in ("rows_flat_kernel", "rows_split_kernel", "draw_kernel"):
            if kn in name:
                short = f"{kn}<{'BF16' if 'BF16' in name else 'F32'}>"
        if short is None or name not in write:
            continue
        rec = {"kernel": short, "workload": "B=64, gamma=5, V=151936, bf16 logits, fp32 q, T=0.8",
               "dispatches": fetch[name][0],
               "fetch_kib_per_dispatch": fetch[name][1], "write_kib_per_dispatch": write[name][1],
               "copy_reference": {"kernel": ck, "bytes": COPY_BYTES,
                                  "fetch_kib": fetch[ck][1], "write_kib": write[ck][1],
                                  "fetch_scale": f_scale, "write_scale": w_scale},
               "bytes_per_launch": int(fetch[name][1] * 1024.0 * f_scale + write[name][1] * 1024.0 * w_scale),
               "fetch_bytes_per_launch": int(fetch[name][1] * 1024.0 * f_scale),
               "write_bytes_per_launch": int(write[name][1] * 1024.0 * w_scale),
               "kernel_source_sha256": sha,
               "sources": {"fetch": os.path.relpath(fetch_csv, ROOT), "write": os.path.relpath(write_csv, ROOT)}}
        with open(traffic_path(short), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{short}: {rec['bytes_per_launch'] / 1e6:.1f} MB per launch -> {traffic_path(short)}")


def sub_batch(inp, b0: int, b1: int):
    """Requests [b0, b1) of ``inp`` as a batch of their own (same layout rules)."""
    import dataclasses
    import numpy as np
    off = inp.draft_offsets
    d0, d1 = int(off[b0]), int(off[b1])
    t0, t1 = d0 + b0, d1 + b1
    cut = lambda a, lo, hi: None if a is None else a[lo:hi]
    return dataclasses.replace(
        inp, batch=b1 - b0, logits=inp.logits[t0:t1], draft_probs=cut(inp.draft_probs, d0, d1),
        draft_ids=inp.draft_ids[d0:d1], temperature=inp.temperature[b0:b1], uniforms=inp.uniforms[b0:b1],
        offsets=None if inp.offsets is None else (np.asarray(off[b0:b1 + 1]) - d0).astype(np.int32),
        topk_ids=cut(inp.topk_ids, d0, d1), topk_probs=cut(inp.topk_probs, d0, d1))


_POOL_INP = None


def _pool_verify(rng):
    import oracle
    b0, b1 = rng
    oracle.verify(sub_batch(_POOL_INP, b0, b1))
    return b1 - b0


def cpu_baseline(inp, budget_s=10.0, max_workers=16):
    """The oracle timed on the host: one process, then forked workers over request
    chunks.  Runs before any GPU call (forking a process that has initialised the
    GPU is not allowed)."""
    import multiprocessing as mp
    import oracle
    global _POOL_INP
    t0 = time.perf_counter()
    n1 = 0
    while True:
        oracle.verify(inp)
        n1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s or n1 >= 50:
            break
    host_cpus = os.cpu_count() or 1
    workers = max(1, min(host_cpus, max_workers, inp.batch))
    bounds = [round(k * inp.batch / workers) for k in range(workers + 1)]
    chunks = [(bounds[k], bounds[k + 1]) for k in range(workers) if bounds[k + 1] > bounds[k]]
    _POOL_INP = inp
    with mp.get_context("fork").Pool(len(chunks)) as pool:
        pool.map(_pool_verify, chunks)             # start-up outside the timing
        t0 = time.perf_counter()
        nw = 0
        while True:
            done = sum(pool.map(_pool_verify, chunks))
            assert done == inp.batch
            nw += 1
            elw = time.perf_counter() - t0
            if elw >= budget_s or nw >= 200:
                break
    _POOL_INP = None
    return {"value": round(nw / elw, 4), "unit": "steps/s", "cores": len(chunks), "kind": "oracle",
            "sample": f"{nw} full B={inp.batch} steps of the same workload, each split into {len(chunks)} "
                      f"request chunks over {len(chunks)} forked worker processes (fp64 NumPy)",
            "host_cpu_count": host_cpus,
            "one_core": {"value": round(n1 / el1, 4), "unit": "steps/s", "cores": 1,
                         "sample": f"{n1} full steps in one process"}}


def durations_path():
    return os.path.join(ROOT, "profiles", "kernel_durations_B64_g5_V151936.json")


def write_durations(stats_csv):
    """Per-kernel average durations of one rocprofv3 --stats run (kernel_stats.csv),
    stamped with the kernel sources' hash, for the bench line's roofline."""
    import csv
    out = {"workload": "B=64, gamma=5, V=151936, bf16 logits, fp32 q, T=0.8",
           "kernel_source_sha256": kernel_source_sha(), "source": os.path.relpath(stats_csv, ROOT), "kernels": {}}
    with open(stats_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Name"]
            for kn in ("rows_flat_kernel", "rows_split_kernel", "draw_kernel"):
                if f"sv::{kn}<" in name:
                    short = f"{kn}<{'BF16' if 'BF16' in name else 'F32'}>"
                    out["kernels"][short] = {"calls": int(row["Calls"]),
                                             "avg_ms": float(row["AverageNs"]) / 1e6,
                                             "min_ms": float(row["MinNs"]) / 1e6,
                                             "max_ms": float(row["MaxNs"]) / 1e6}
    with open(durations_path(), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["kernels"], indent=1))


def profiled_avg_ms(kernel: str):
    """rocprofv3's average duration of ``kernel`` on this workload, if recorded for
    the current kernel sources."""
    try:
        rec = json.load(open(durations_path()))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    k = rec["kernels"].get(kernel)
    return None if k is None else k["avg_ms"]


# Read-probe layouts the ceiling is taken over: (name, mode, workgroups per CU).
# Grid-stride (the grid reads one dense window at a time) is the fastest form on
# this device; spans (one contiguous range per workgroup, the rows kernel's
# layout) and chunks (contiguous chunks interleaved over the grid) for context.
CEILING_LAYOUTS = (("stride8nt", 0, 1), ("stride8nt", 0, 3), ("stride8nt", 0, 6), ("stride8nt", 0, 8),
                   ("stride16nt", 4, 3), ("stride16nt", 4, 8), ("span8nt", 1, 3), ("chunk8nt", 8, 3))


def read_ceiling(torch, nbytes_list, reps=5):
    """Streaming-read GB/s per probe layout over buffers of the given sizes: the
    median of ``reps`` launches, each on a different buffer of a set larger than
    the Infinity Cache, so that no launch reads what the previous one left there.
    Returns {nbytes: {layout: GB/s}}."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "lossless_rejection_sampling_sampler_amd", "libhbmprobe.so"))
    lib.hbm_read_probe_time.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    lib.hbm_read_probe_time.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(16 * cus, dtype=torch.int32, device="cuda:0")
    res = {}
    for nb in nbytes_list:
        nb = nb // 16 * 16
        bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda:0") for _ in range(max(2, (320 << 20) // nb + 1))]
        for b in bufs:
            b.fill_(1)
        torch.cuda.synchronize()
        row = {}
        for name, mode, per in CEILING_LAYOUTS:
            times = []
            for r in range(reps):
                b = bufs[r % len(bufs)]
                ms = ctypes.c_float()
                st = lib.hbm_read_probe_time(ctypes.c_void_p(b.data_ptr()), nb, ctypes.c_void_p(out.data_ptr()),
                                             per * cus, mode, 1 if r == 0 else 0, 1, ctypes.byref(ms))
                if st:
                    raise RuntimeError(f"hbm_read_probe_time status {st}")
                times.append(ms.value)
            times.sort()
            row[f"{name}_{per}perCU"] = round(nb / (times[len(times) // 2] * 1e-3) / 1e9, 1)
        res[nb] = row
        del bufs
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--rotate", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds per CPU baseline leg")
    ap.add_argument("--seed-replicate", type=int, default=0)
    ap.add_argument("--workload", choices=list(WORKLOAD_TEXT), default="config3",
                    help="config3 (the default line); other workloads are for comparison runs")
    ap.add_argument("--schedule", choices=["auto", "twokernel"], default="auto",
                    help="rows + draw kernels, or the library's choice")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (one call per replay, "
                         "input sets rotating) and report it as graph_steps_per_s")
    ap.add_argument("--profile-steps", type=int, default=500,
                    help="steps of the dispatch-stamped per-kernel timing pass")
    ap.add_argument("--dist-steps", type=int, default=500,
                    help="steps of the per-step timing pass (median / p10 / p90)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="for rocprofv3 counter passes: a plain copy of known size (the scale "
                         "reference), then --warmup + --steps verify steps; prints no JSON")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="(CPU only) turn two counter_collection.csv files of --pmc-workload runs "
                         "into per-kernel HBM traffic records under profiles/")
    ap.add_argument("--durations-from", metavar="KERNEL_STATS_CSV",
                    help="(CPU only) record rocprofv3's per-kernel averages of a default-workload run "
                         "under profiles/ for the bench line")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.durations_from:
        write_durations(args.durations_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the verify step shards by "
              "request with no exchange, so N GPUs run N independent copies of this step.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np

    log(f"[bench] generating workload {args.workload}")
    inp = make_workload(args.workload, args.seed_replicate)
    wl_text = WORKLOAD_TEXT[args.workload]
    cpu = None
    if not args.no_cpu_baseline and not args.pmc_workload:
        log("[bench] timing the CPU oracle (before any GPU call)")
        cpu = cpu_baseline(inp, args.cpu_budget)
        log(f"[bench] oracle: {cpu['one_core']['value']} steps/s on one core, {cpu['value']} on {cpu['cores']}")

    import torch

    from lossless_rejection_sampling_sampler_amd import SpecVerify, upload
    from lossless_rejection_sampling_sampler_amd._lib import SCHEDULE_NAMES

    dev = torch.device("cuda:0")
    log("[bench] uploading, rotate=%d" % args.rotate)
    base = upload(logits=inp.logits, logits_dtype=inp.dtype, draft_probs=inp.draft_probs,
                  draft_ids=inp.draft_ids, temperature=inp.temperature, uniforms=inp.uniforms,
                  gamma=inp.gamma, draft_offsets=inp.offsets, device=dev,
                  topk_ids=inp.topk_ids, topk_probs=inp.topk_probs)
    copies = [base]
    for _ in range(args.rotate - 1):
        c = upload(logits=inp.logits[:1], logits_dtype=inp.dtype,
                   draft_probs=None if inp.draft_probs is None else inp.draft_probs[:1],
                   draft_ids=inp.draft_ids, temperature=inp.temperature, uniforms=inp.uniforms,
                   gamma=inp.gamma, draft_offsets=inp.offsets, device=dev,
                   topk_ids=inp.topk_ids, topk_probs=inp.topk_probs)
        c.target_logits = base.target_logits.clone()
        if base.draft_probs is not None:
            c.draft_probs = base.draft_probs.clone()
        copies.append(c)
    torch.cuda.synchronize()

    schedule = None if args.schedule == "auto" else args.schedule
    if args.pmc_workload:
        # the scale reference: an elementwise copy reading and writing COPY_BYTES each
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    sv = SpecVerify(inp.batch, inp.gamma, inp.vocab, inp.dtype, device=0, schedule=schedule)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # argument blocks are built once so the timed loop is one C call per step
    packed = [c.args() for c in copies]

    def step(ctx, i):
        st = ctx.run_args(packed[i % len(packed)], sh)
        if st:
            raise RuntimeError(f"spec_verify_run failed with status {st}")

    for i in range(args.warmup):
        step(sv, i)
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({args.warmup} steps); timing {args.steps} steps")

    # ---- timed region: exactly K steps, synchronised on both sides
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(sv, i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    log(f"[bench] {ms_per_step * 1e3:.2f} us per step")

    if args.pmc_workload:
        log(f"[bench] counter workload done: {args.warmup + args.steps} steps")
        sv.close()
        return

    # ---- per-step times: one event between consecutive steps
    nd = max(2, args.dist_steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nd + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(nd):
        step(sv, i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(nd)])
    dist = {"steps": nd, "median_ms": round(float(np.median(per)), 6),
            "p10_ms": round(float(np.percentile(per, 10)), 6), "p90_ms": round(float(np.percentile(per, 90)), 6),
            "mean_ms": round(float(per.mean()), 6)}

    graph_rate = graph_multi_rate = None
    if args.graph:
        # one captured call per input set; replays cycle through them
        graphs = []
        for i in range(len(packed)):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                # launched on the capture stream torch has made current
                st = sv.run_args(packed[i], torch.cuda.current_stream().cuda_stream)
                if st:
                    raise RuntimeError(f"spec_verify_run failed with status {st} under capture")
            graphs.append(gph)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_rate = 1000.0 * args.steps / g0.elapsed_time(g1)
        # the same calls, GRAPH_CALLS of them per captured graph (one replay
        # launches them all): separates the replay's own launch cost from the
        # kernels'
        big = torch.cuda.CUDAGraph()
        with torch.cuda.graph(big):
            for i in range(GRAPH_CALLS):
                st = sv.run_args(packed[i % len(packed)], torch.cuda.current_stream().cuda_stream)
                if st:
                    raise RuntimeError(f"spec_verify_run failed with status {st} under capture")
        torch.cuda.synchronize()
        reps = max(1, args.steps // GRAPH_CALLS)
        for i in range(max(1, args.warmup // GRAPH_CALLS)):
            big.replay()
        torch.cuda.synchronize()
        g0.record(stream)
        for i in range(reps):
            big.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_multi_rate = 1000.0 * reps * GRAPH_CALLS / g0.elapsed_time(g1)

    sv_schedule = sv.last_schedule()
    tok, num = base.results()
    for c in copies[1:]:
        t2, n2 = c.results()
        assert np.array_equal(n2, num) and np.array_equal(t2, tok), "rotated copies disagree"
    rows_b, draw_b = algorithmic_bytes(inp, num)
    step_bytes = rows_b + draw_b

    # ---- per-kernel durations, stamped by the kernels' own dispatches
    svp = SpecVerify(inp.batch, inp.gamma, inp.vocab, inp.dtype, device=0, profile=True, schedule=schedule)
    for i in range(args.warmup):
        step(svp, i)
    torch.cuda.synchronize()
    svp.profile_read()
    kp = max(1, args.profile_steps)
    for i in range(kp):
        step(svp, i)
    rows_ms, draw_ms, n_prof = svp.profile_read()
    rows_avg_ms, draw_avg_ms = rows_ms / n_prof, draw_ms / n_prof
    svp.close()
    log(f"[bench] kernels: rows {rows_avg_ms * 1e3:.2f} us, draw {draw_avg_ms * 1e3:.2f} us")

    ceiling = None
    if not args.no_ceiling:
        for c in copies[1:]:
            c.target_logits = c.draft_probs = None
        copies = copies[:1]
        packed = packed[:1]
        torch.cuda.empty_cache()
        cz = read_ceiling(torch, [1 << 30, step_bytes])
        big, small = cz[(1 << 30) // 16 * 16], cz[step_bytes // 16 * 16]
        ceiling = {"read_1GiB_gbps": max(big.values()), "read_step_bytes_gbps": max(small.values()),
                   "best_layout_1GiB": max(big, key=big.get), "best_layout_step_bytes": max(small, key=small.get),
                   "layouts_1GiB_gbps": big, "layouts_step_bytes_gbps": small,
                   "kernel": "16-byte loads; median of 5 launches, each on another buffer (set > Infinity Cache)"}
        log(f"[bench] read ceiling {ceiling}")

    def roofline(kname, kbytes, kms):
        gbps = kbytes / (kms * 1e-3) / 1e9
        prof = profiled_avg_ms(kname) if args.workload == "config3" else None
        r = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(gbps / PEAK_HBM_GBPS, 4), "kernel": kname, "bytes_per_launch": kbytes,
             "avg_launch_ms": round(kms, 6), "timing": "dispatch-stamped HIP events over the profiling pass",
             "traffic": traffic_entry(kname) if args.workload == "config3" else None,
             "rocprof_avg_ms": prof,
             "rocprof_frac": None if prof is None else round(kbytes / (prof * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        return r

    split = sv_schedule == 1
    lines = [roofline(f"{'rows_split_kernel' if split else 'rows_flat_kernel'}<{KDT if inp.dtype == 'bf16' else 'F32'}>",
                      rows_b, rows_avg_ms),
             roofline(f"draw_kernel<{KDT if inp.dtype == 'bf16' else 'F32'}>", draw_b, draw_avg_ms)]
    dominant = max(lines, key=lambda r: r["avg_launch_ms"])
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    sampled = inp.temperature > 0
    gam = inp.gammas
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; f32 exp + f64 sums; f64 draw",
        "data": "synthetic (seeded; shapes of the pages' gamma=5, T=0.8 deployment)",
        "config": {"workload": f"verify step {inp.name}: {wl_text}", "batch": inp.batch, "gamma": inp.gamma,
                   "vocab": inp.vocab, "rotating_input_sets": args.rotate},
        "hbm_gbps": round(step_gbps, 1),
        "frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "step_time_distribution": dist,
        "schedule": SCHEDULE_NAMES.get(sv_schedule, "none"),
        "kernels": {"rows_ms": round(rows_avg_ms, 6), "draw_ms": round(draw_avg_ms, 6),
                    "rows_bytes": rows_b, "draw_bytes": draw_b, "profiled_steps": n_prof},
        "acceptance": {"mean_accepted": float(num.mean()),
                       "residual_draws": int((sampled & (num < gam)).sum()),
                       "bonus_draws": int((sampled & (num == gam)).sum())},
        "graph_steps_per_s": None if graph_rate is None else round(graph_rate, 2),
        "graph_steps_per_s_multi": None if graph_multi_rate is None else
            {"calls_per_graph": GRAPH_CALLS, "value": round(graph_multi_rate, 2)},
        "read_ceiling": ceiling,
        "roofline": dominant,
        "roofline_per_kernel": lines,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    sv.close()


if __name__ == "__main__":
    main()
