#!/usr/bin/env python3
"""Decode-phase paged attention on one MI355X: KV-read GB/s and us/step.

One step is one decode_attn call over the whole batch: one layer's decode attention
(the main kernel, plus the merge kernel when the plan cuts segments). The default
workload is the largest single-GPU preset, the Llama-3-8B-shaped GQA batch: batch 160,
32 query heads over 8 KV heads (group 4), head_dim 128, seq_lens uniform in [64, 4096],
16-token pages in a shuffled pool, fp16 K/V ~ N(0, 1). --config picks another preset.

Inputs are resident in HBM before timing starts. To keep the 256 MB Infinity Cache from
serving the KV reads, the step rotates over R replicas of the page pools totalling at
least 1 GiB. Throughput counts algorithmic KV bytes only: sum_b L_b * Hkv * 2 * D * elem
(plus the fp32 row scales for INT8 and FP8).

Timing: W warm-up steps (continued until at least 0.25 s of GPU work has run, so that the
clocks are up), then `repeats` windows of exactly --steps back-to-back steps,
each between one pair of HIP events on the launch stream with a device synchronisation
on both sides. `value` and `us_per_step` are the median window; the spread is reported.

Prints one JSON line on stdout; progress goes to stderr. --op append, prefill and step
time the other entry points on their workloads; --op hbm measures the reference reads
(decode_attn_hbm_reference) on the workload's tiles: the attainable HBM rate that the
roofline record's `attainable` field compares the step with.

    python bench.py --summarize-profile DIR --tag TAG

turns the rocprofv3 CSVs of one profiled workload (kernel trace, FETCH_SIZE, WRITE_SIZE
and the counter passes, in the directory layout the summary lists) into
profiles/<op>_<workload>.txt (for --op hbm, the kernel trace alone into
profiles/hbm_reference_<workload>.txt).
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published peak
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak, published
METRIC = "decode-attn KV-read GB/s (fraction of MI355X HBM peak) + µs/step"
PROFILES = os.path.join(ROOT, "profiles")
DEFAULT_CONFIG = {"attn": 3, "append": 2, "step": 2, "prefill": 8, "hbm": 3}
MIN_WARMUP_S = 0.25   # least GPU work before the timed windows (clocks up after idling)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ATTN_SOURCES = ("api.cpp", "kernels.h", "kernels.hip")
APPEND_SOURCES = ("api.cpp", "kernels.h", "append.hip")
PREFILL_SOURCES = ("api.cpp", "kernels.h", "prefill.hip")
STEP_SOURCES = ("api.cpp", "kernels.h", "kernels.hip", "append.hip")
HBM_SOURCES = ("api.cpp", "kernels.h", "hbm_reference.hip")
SOURCES_OF_OP = {"attn": ATTN_SOURCES, "append": APPEND_SOURCES, "prefill": PREFILL_SOURCES,
                 "step": STEP_SOURCES, "hbm": HBM_SOURCES}
PREFIX_OF_OP = {"attn": "decode_attn", "append": "decode_attn_append",
                "prefill": "decode_attn_prefill", "step": "decode_attn_step",
                "hbm": "hbm_reference"}


def strip_comments(text: str) -> str:
    """C++ source without its comments and blank lines, trailing spaces trimmed; string and
    character literals are kept whole (a // inside one is not a comment)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            end = text.find("*/", i + 2)
            i = n if end < 0 else end + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(sources=ATTN_SOURCES) -> str:
    """Hash of the sources that decide what a kernel does (the kernel file, the internal
    interface and the host side that plans and launches it), without their comments: an
    edit of a comment leaves the compiled kernels, and so the profiles, as they were."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_phase_attention_paged_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def read_profile(workload_name: str, op: str = "attn"):
    """The committed rocprofv3 summary of a workload as a dict of its top-level fields, or
    (None, reason) when there is none or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"{PREFIX_OF_OP[op]}_{workload_name}.txt")
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
    if fields.get("kernel_source_sha256") != kernel_source_hash(SOURCES_OF_OP[op]):
        return None, "kernel changed since the counters were taken"
    fields["_path"] = os.path.relpath(path, ROOT)
    return fields, path


def profile_traffic(fields):
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, TypeError, ValueError):
        return None


def host_info():
    """Cores this process may run on and the host CPU model."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cores, model


class _ThreadLimit:
    """BLAS/OpenMP threads of the oracle's NumPy set to `n` (when threadpoolctl exists)."""

    def __init__(self, n):
        self.n, self.ctx = n, None

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self.ctx = threadpool_limits(limits=self.n)
            self.ctx.__enter__()
        except Exception:  # pragma: no cover
            self.ctx = None
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)


def cpu_baseline(w, budget_s: float = 10.0):
    """The fp64 oracle as it stands, timed on the host over a bounded sample: a prefix of
    the batch sized to about `budget_s` seconds, repeated while the budget lasts."""
    import numpy as np
    import oracle
    from decode_phase_attention_paged_amd.workload import ELEM_BYTES, SCALE_BYTES, kv_read_bytes
    cores, model = host_info()
    c = w.config
    with _ThreadLimit(cores):
        t0 = time.perf_counter()
        oracle.decode_attention(w.q[:1], w.k_pages, w.v_pages, w.block_table[:1], w.seq_lens[:1],
                                w.scale, w.k_scale, w.v_scale)
        per_token = max((time.perf_counter() - t0) / max(int(w.seq_lens[0]), 1), 1e-9)
        total_tokens = int(w.seq_lens.sum())
        n = c.batch
        if per_token * total_tokens > budget_s:
            cum = np.cumsum(w.seq_lens.astype(np.int64))
            n = max(1, int(np.searchsorted(cum, budget_s / per_token)))
        sample_bytes = kv_read_bytes(w.seq_lens[:n], c.n_kv_heads, c.head_dim,
                                     ELEM_BYTES[c.kv_dtype], SCALE_BYTES[c.kv_dtype])
        reps, spent = 0, 0.0
        while reps < 1 or (spent < budget_s and reps < 50):
            t0 = time.perf_counter()
            oracle.decode_attention(w.q[:n], w.k_pages, w.v_pages, w.block_table[:n],
                                    w.seq_lens[:n], w.scale, w.k_scale, w.v_scale)
            spent += time.perf_counter() - t0
            reps += 1
    gbs = sample_bytes * reps / spent / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} of {c.batch} sequences x {reps} repetitions "
                      f"({sample_bytes * reps / 1e9:.3f} GB of KV in {spent:.1f} s); NumPy "
                      f"float64, BLAS threads limited to the {cores} cores of this "
                      f"process's affinity mask",
            "cpu_model": model,
            "seconds_per_full_step": round(spent / reps * total_tokens /
                                           max(int(w.seq_lens[:n].sum()), 1), 4)}


def copy_calibration(torch, nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH/WRITE counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


# Arithmetic type named in the JSON line, by KV storage format (the kernels accumulate in fp32
# whatever the storage type).
DTYPE_NAMES = {"fp16": "f16", "bf16": "bf16", "int8": "i8", "fp8": "fp8e4m3"}


def device_tensor(torch, np, a, dev):
    """A host array on the GPU; bf16 bit patterns (uint16) become bfloat16 tensors and E4M3
    codes (uint8) float8_e4m3fn tensors."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    t = torch.from_numpy(a).to(dev)
    return t.view(torch.float8_e4m3fn) if a.dtype == np.uint8 else t


def replicas_for(args, pool_bytes: int) -> int:
    reps = args.replicas or max(2, math.ceil((1 << 30) / pool_bytes))
    return min(reps, max(1, (48 << 30) // pool_bytes))


def timed_windows(torch, stream, step, steps: int, windows: int, first: int):
    """`windows` timed windows of exactly `steps` back-to-back calls of step(i), each
    between one pair of HIP events recorded on `stream` (the stream the library launches
    on), with a device synchronisation before and after. No event sits between steps: an
    event record between two launches delays the second one by several microseconds on
    this GPU. Returns (ms per window, host wall seconds per window)."""
    total_ms, walls = [], []
    i = first
    for _ in range(windows):
        start_ev = torch.cuda.Event(enable_timing=True)
        stop_ev = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start_ev.record(stream)
        for _ in range(steps):
            step(i)
            i += 1
        stop_ev.record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - wall0)
        total_ms.append(start_ev.elapsed_time(stop_ev))
    return total_ms, walls


def window_stats(total_ms, steps):
    per = sorted(t / steps for t in total_ms)
    return {"median_ms": statistics.median(per), "min_ms": per[0], "max_ms": per[-1]}


def default_windows(steps: int) -> int:
    """At least five windows and at least 100 timed steps in all."""
    return max(5, math.ceil(100 / max(steps, 1)))


# Kernels one step launches, by plan mode (stream, split, segment).
def kernel_names(mode: int, kv: str, group: int):
    t = f"<{kv},G={group}>"
    return {0: [f"stream_kernel{t}", "piece_merge_kernel"],
            1: [f"split_kernel{t}", "split_merge_kernel"],
            2: [f"seg_kernel{t}"]}[mode]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--repeats", type=int, default=0,
                    help="timed windows of --steps steps each (0 = max(5, ceil(100/steps)))")
    ap.add_argument("--config", type=int, default=0, choices=list(range(12)),
                    help="workload preset (0 = the op's default: 3 for attn, 2 for append "
                         "and step, 8 for prefill)")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="stream mode on this many workgroups, or the grid of segment mode "
                         "with --splits 1 (0 = the library's plan)")
    ap.add_argument("--splits", type=int, default=0,
                    help="1 = segment mode, >1 = split mode with this many partitions "
                         "(0 = the library's plan)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >= 1 GiB")
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="keep warming up until this much GPU work has run (0 for profiled runs)")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the labelled one-replica (hot pool) figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--graph", type=int, default=0,
                    help="capture this many consecutive steps in one HIP graph and time "
                         "replays of it (the step count is rounded up to a multiple)")
    ap.add_argument("--kv", choices=["fp16", "bf16", "int8", "fp8"], default=None,
                    help="run the preset's shapes over another storage format (the workload "
                         "name gets the format as a suffix)")
    ap.add_argument("--op", choices=["attn", "append", "prefill", "step", "hbm"], default="attn",
                    help="attn: the decode-attention step (default); append: the K/V append "
                         "that precedes it in a decode step, on the same workload; step: "
                         "append then attention; prefill: chunked-prefill attention; hbm: "
                         "reference read rates for the roofline, on the workload's tiles")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="write profiles/<op>_<workload>.txt from the rocprofv3 CSVs in DIR")
    ap.add_argument("--tag", default=None, help="with --summarize-profile: the run's tag")
    args = ap.parse_args()

    if args.summarize_profile:
        if not args.tag:
            ap.error("--summarize-profile needs --tag")
        summarize_profile(args.summarize_profile, args.tag)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library runs decode attention on a single "
              "MI355X, and multi-GPU sharding is a design note only; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.repeats <= 0:
        args.repeats = default_windows(args.steps)

    import numpy as np
    import torch
    from decode_phase_attention_paged_amd import binding
    from decode_phase_attention_paged_amd.workload import CONFIGS, generate

    if args.copy_calibration:
        copy_calibration(torch)
        return

    lib = binding.load_library()
    if args.config == 0:
        args.config = DEFAULT_CONFIG[args.op]
    cfg = CONFIGS[args.config]
    if args.kv and args.kv != cfg.kv_dtype:
        cfg = cfg.with_(kv_dtype=args.kv, name=f"{cfg.name}_{args.kv}")
    if args.op == "append":
        return bench_append(args, cfg, lib, torch, np, binding, generate)
    if args.op == "prefill":
        return bench_prefill(args, cfg, lib, torch, np, binding, generate)
    if args.op == "step":
        return bench_step(args, cfg, lib, torch, np, binding, generate)
    if args.op == "hbm":
        return bench_hbm(args, cfg, torch, np, binding)
    log(f"generating {cfg.name} ...")
    w = generate(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: device_tensor(torch, np, a, dev)
    q, bt, sl = t(w.q), t(w.block_table), t(w.seq_lens)
    pool_bytes = 2 * w.k_pages.nbytes + (2 * w.k_scale.nbytes if w.k_scale is not None else 0)
    reps = replicas_for(args, pool_bytes)
    pools = []
    for _ in range(reps):
        pools.append((t(w.k_pages), t(w.v_pages), t(w.k_scale), t(w.v_scale)))
    out = torch.empty(w.q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    kv_type = binding._KV_CODES[cfg.kv_dtype]
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan = binding.plan(cfg.batch, cfg.max_blocks_per_seq, cfg.n_q_heads, cfg.n_kv_heads,
                        cfg.block_size, cfg.kv_dtype, args.workgroups, args.splits, num_cus)
    explicit = bool(args.workgroups or args.splits)
    group = cfg.n_q_heads // cfg.n_kv_heads
    kernels = kernel_names(plan.mode, cfg.kv_dtype, group)

    # Marshal the arguments once; the timed loop calls the C ABI directly.
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    s_handle = ctypes.c_void_p(stream.cuda_stream)
    call_args = []
    workspace = None
    if explicit and plan.workspace_bytes:
        workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    for kp, vp, ks, vs in pools:
        common = (p(q), p(kp), p(vp), p(ks), p(vs), p(bt), p(sl), cfg.batch,
                  cfg.max_blocks_per_seq, w.num_pages, cfg.n_q_heads, cfg.n_kv_heads,
                  cfg.head_dim, cfg.block_size, kv_type, float(w.scale), p(out))
        if explicit:
            call_args.append(("ex", common + (None, args.workgroups, args.splits, p(workspace),
                                              ws_bytes, s_handle)))
        else:
            call_args.append(("auto", common + (s_handle,)))

    def call(kind, a):
        st = lib.decode_attn(*a) if kind == "auto" else lib.decode_attn_ex(*a)
        if st != 0:
            raise RuntimeError(f"decode_attn failed: {binding.STATUS.get(st, st)}")

    rotate = lambda i: call(*call_args[i % reps])
    hot = lambda i: call(*call_args[0])

    log(f"plan: {plan} replicas={reps} "
        f"pool={pool_bytes / 1e6:.1f} MB kv_bytes/step={w.kv_bytes / 1e6:.1f} MB")
    args.warmup_run = warm_up(torch, rotate, args.warmup, args.min_warmup_s)

    step = rotate
    if args.graph > 0:
        # The same calls, recorded on a capture stream, args.graph steps per graph; replays
        # run on torch's current stream, where the events are recorded.
        cap = torch.cuda.Stream()
        handle = ctypes.c_void_p(cap.cuda_stream)
        captured = [(kind, a[:-1] + (handle,)) for kind, a in call_args]
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.graph):
                call(*captured[i % reps])
        torch.cuda.synchronize()
        args.steps = -(-args.steps // args.graph) * args.graph
        graph.replay()
        torch.cuda.synchronize()
        log(f"graph: {args.graph} steps per replay")
        replays = args.steps // args.graph
        step = lambda i: graph.replay()
        steps_per_window, scale_steps = replays, args.graph
    else:
        steps_per_window, scale_steps = args.steps, 1

    total_ms, walls = timed_windows(torch, stream, step, steps_per_window, args.repeats,
                                    args.warmup_run)
    st = window_stats(total_ms, steps_per_window * scale_steps)
    ms_per_step = st["median_ms"]
    gbs = w.kv_bytes / (ms_per_step / 1e3) / 1e9
    log(f"{args.repeats} windows x {args.steps} steps: us/step median {ms_per_step * 1e3:.2f} "
        f"[{st['min_ms'] * 1e3:.2f}, {st['max_ms'] * 1e3:.2f}]  GB/s={gbs:.1f} "
        f"({gbs / HBM_PEAK_GBS:.4f} of peak)")
    if max(walls) * 1e3 > 1.5 * max(total_ms):
        log("warning: host launch rate may be limiting the step rate")

    hot_rec = None
    if not args.no_hot and args.graph == 0:
        warm_up(torch, hot, args.warmup, args.min_warmup_s)
        hot_ms, _ = timed_windows(torch, stream, hot, args.steps, args.repeats, 0)
        hs = window_stats(hot_ms, args.steps)
        hot_rec = {"us_per_step": round(hs["median_ms"] * 1e3, 3),
                   "gbs": round(w.kv_bytes / (hs["median_ms"] / 1e3) / 1e9, 2),
                   "replicas": 1,
                   "note": "hot: every step reads the same pool replica, so up to 256 MB of it "
                           "may be served by the Infinity Cache; not the headline"}
        log(f"hot (one replica): us/step {hot_rec['us_per_step']} GB/s {hot_rec['gbs']}")

    prof, prof_src = read_profile(cfg.name, "attn")
    traffic = profile_traffic(prof) if prof else None
    log(f"profile: {prof_src}")
    ref, _ = read_profile(cfg.name, "hbm")
    baseline = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        baseline = cpu_baseline(w)
        log(f"cpu baseline: {baseline}")

    launches = len(kernels)
    # One launch per step: the step time is that kernel's average launch duration
    # (back-to-back launches leave no gap). Two launches: the step time is the sum of both,
    # a conservative stand-in for the main kernel's duration, which the profile splits out.
    achieved = w.kv_bytes / (ms_per_step / 1e3) / 1e9
    record = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": getattr(args, "warmup_run", args.warmup),
        "repeats": args.repeats,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_min_max": [round(st["min_ms"] * 1e3, 3), round(st["max_ms"] * 1e3, 3)],
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
        "argv": sys.argv[1:],
        "config": {
            "workload": cfg.name,
            "batch": cfg.batch, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
            "head_dim": cfg.head_dim, "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
            "seq_lens": f"uniform [{cfg.len_lo}, {cfg.len_hi}], seed {w.seed}",
            "tokens": int(w.seq_lens.sum()), "num_pages": w.num_pages,
            "plan": {"mode": binding._MODE_NAMES[plan.mode],
                     "workgroups": plan.num_workgroups, "splits": plan.num_splits},
            "replicas": reps,
            "graph_steps": args.graph,
            "kv_bytes_per_step": int(w.kv_bytes),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernels[0],
            "launches_per_step": launches,
            "avg_launch_us": round(ms_per_step * 1e3, 3) if launches == 1 else None,
            "step_us": round(ms_per_step * 1e3, 3),
            "achieved_from": "median step time (= the kernel's launch duration)" if launches == 1
                             else "median step time of both launches (conservative)",
            "profile": None if not prof else {
                "file": prof["_path"],
                "dominant_kernel_avg_us": round(float(prof["dominant_kernel_timed_avg_ns"]) / 1e3, 3),
                "traffic_over_algorithmic": float(prof["traffic_over_algorithmic"]),
            },
            "attainable": None if not ref else {
                "what": "best rate of a plain random gather of the same step's K/V tiles "
                        "(bench.py --op hbm)",
                "gbs": float(ref["best_gather_gbs"]),
                "frac": round(achieved / float(ref["best_gather_gbs"]), 4),
                "file": ref["_path"],
            },
        },
        "hot": hot_rec,
        "cpu_baseline": baseline,
    }
    print(json.dumps(record), flush=True)


def append_bytes(batch: int, n_kv_heads: int, head_dim: int, kv_dtype: str) -> int:
    """Algorithmic bytes of one append launch that writes every row: the new K and V rows
    read (16-bit), the stored rows written (16-bit, or 8-bit codes plus an fp32 row scale),
    and each sequence's position and block-table entry read."""
    rows = batch * n_kv_heads
    written = head_dim * 2 if kv_dtype in ("fp16", "bf16") else head_dim + 4
    return rows * 2 * (head_dim * 2 + written) + batch * 8


def append_cpu_baseline(w, table, positions, new, budget_s: float = 10.0):
    """oracle.append_kv as it stands, timed on the host over whole launches."""
    import oracle
    c = w.config
    cores, model = host_info()
    reps, spent = 0, 0.0
    with _ThreadLimit(cores):
        while reps < 1 or (spent < budget_s and reps < 200):
            t0 = time.perf_counter()
            oracle.append_kv(w.k_pages, w.v_pages, table, positions, new[0], new[1],
                             c.block_size, w.k_scale, w.v_scale)
            spent += time.perf_counter() - t0
            reps += 1
    nbytes = append_bytes(c.batch, c.n_kv_heads, c.head_dim, c.kv_dtype)
    return {"value": round(nbytes * reps / spent / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{reps} whole launches ({c.batch * c.n_kv_heads} rows each) in "
                      f"{spent:.1f} s, pool copies included"}


def grow_for_append(w, np, cfg):
    """Positions L_b for every sequence's next token, with a fresh page (numbered past the
    pool) where that token starts one. Returns (table, positions, fresh)."""
    table = w.block_table.copy()
    positions = w.seq_lens.astype(np.int32).copy()
    fresh = 0
    for b in range(cfg.batch):
        j = int(positions[b]) // cfg.block_size
        if j >= table.shape[1]:
            positions[b] = int(positions[b]) - 1      # a full table: rewrite the last slot
        elif table[b, j] < 0:
            table[b, j] = w.num_pages + fresh
            fresh += 1
    return table, positions, fresh


def warm_up(torch, step, warmup: int, min_s: float = MIN_WARMUP_S) -> int:
    """`warmup` untimed steps, then more until at least `min_s` seconds of GPU work have run:
    after the host-side data generation the GPU has idled for seconds, and its clocks take
    tens of milliseconds of load to come back up. Returns the number of steps run.""" 
    t0 = time.perf_counter()
    i = 0
    while i < warmup:
        step(i)
        i += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(16):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return i


def timed_record(args, torch, stream, step, nbytes):
    """Warm-up, then the timed windows; returns (median ms/step, stats)."""
    args.warmup_run = warm_up(torch, step, args.warmup, args.min_warmup_s)
    total_ms, _ = timed_windows(torch, stream, step, args.steps, args.repeats, args.warmup_run)
    st = window_stats(total_ms, args.steps)
    return st["median_ms"], st


def bench_append(args, cfg, lib, torch, np, binding, generate):
    """Time decode_attn_append: every sequence of the workload writes its next token
    (position L_b) into its page slot; sequences whose next token starts a new page get a
    fresh page. The new rows are fp16 ~ N(0, 1) scaled per row by U(0.1, 10)."""
    log(f"generating {cfg.name} for the append ...")
    w = generate(cfg)
    table, positions, fresh = grow_for_append(w, np, cfg)
    n_pages = w.num_pages + fresh
    rng = np.random.default_rng(w.seed + 1)
    shape = (cfg.batch, cfg.n_kv_heads, cfg.head_dim)
    new = [(rng.standard_normal(shape, dtype=np.float32) *
            rng.uniform(0.1, 10, size=shape[:2] + (1,))).astype(np.float32) for _ in range(2)]
    new = [(x.view(np.uint32) >> 16).astype(np.uint16) if cfg.kv_dtype == "bf16"
           else x.astype(np.float16) for x in new]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scaled = cfg.kv_dtype in ("int8", "fp8")
    pool_shape = (n_pages, cfg.n_kv_heads, cfg.block_size, cfg.head_dim)
    elem = {"fp16": torch.float16, "bf16": torch.bfloat16, "int8": torch.int8,
            "fp8": torch.float8_e4m3fn}[cfg.kv_dtype]
    pool_bytes = 2 * n_pages * cfg.n_kv_heads * cfg.block_size * (
        cfg.head_dim * (1 if scaled else 2) + (4 if scaled else 0))
    reps = replicas_for(args, pool_bytes)
    t = lambda a: device_tensor(torch, np, a, dev)
    bt, pos = t(table), t(positions)
    sets = []
    for _ in range(reps):
        kp = torch.zeros(pool_shape, dtype=torch.uint8 if scaled else torch.int16,
                         device=dev).view(elem)
        vp = torch.zeros_like(kp)
        ks = torch.zeros(pool_shape[:3], dtype=torch.float32, device=dev) if scaled else None
        vs = torch.zeros(pool_shape[:3], dtype=torch.float32, device=dev) if scaled else None
        sets.append((t(new[0]), t(new[1]), kp, vp, ks, vs))
    stream = torch.cuda.current_stream(dev)
    s_handle = ctypes.c_void_p(stream.cuda_stream)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    kv_type = binding._KV_CODES[cfg.kv_dtype]
    call_args = [(p(kn), p(vn), p(bt), p(pos), cfg.batch, cfg.max_blocks_per_seq, n_pages,
                  cfg.n_kv_heads, cfg.head_dim, cfg.block_size, kv_type, p(kp), p(vp), p(ks),
                  p(vs), s_handle) for kn, vn, kp, vp, ks, vs in sets]

    def step(i):
        st = lib.decode_attn_append(*call_args[i % reps])
        if st != 0:
            raise RuntimeError(f"decode_attn_append failed: {binding.STATUS.get(st, st)}")

    nbytes = append_bytes(cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.kv_dtype)
    log(f"append: rows={cfg.batch * cfg.n_kv_heads} fresh_pages={fresh} replicas={reps} "
        f"bytes/launch={nbytes}")
    ms_per_step, st = timed_record(args, torch, stream, step, nbytes)
    gbs = nbytes / (ms_per_step / 1e3) / 1e9
    log(f"us/launch median {ms_per_step * 1e3:.2f} GB/s={gbs:.1f}")
    prof, prof_src = read_profile(cfg.name, "append")
    traffic = profile_traffic(prof) if prof else None
    log(f"profile: {prof_src}")
    baseline = None
    if not args.no_cpu_baseline:
        w_host = w
        if fresh:
            grow = lambda a, fill: None if a is None else np.concatenate(
                [a, np.full((fresh,) + a.shape[1:], fill, dtype=a.dtype)])
            w_host = type(w)(**{**w.__dict__, "k_pages": grow(w.k_pages, 0),
                                "v_pages": grow(w.v_pages, 0), "k_scale": grow(w.k_scale, 0),
                                "v_scale": grow(w.v_scale, 0)})
        baseline = append_cpu_baseline(w_host, table, positions, new)
        log(f"cpu baseline: {baseline}")
    record = {
        "metric": "decode K/V append GB/s (fraction of MI355X HBM peak) + µs/launch",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": getattr(args, "warmup_run", args.warmup),
        "repeats": args.repeats,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_min_max": [round(st["min_ms"] * 1e3, 3), round(st["max_ms"] * 1e3, 3)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp16": "f16", "bf16": "bf16", "int8": "f16->i8",
                  "fp8": "f16->fp8e4m3"}[cfg.kv_dtype],
        "data": "synthetic",
        "argv": sys.argv[1:],
        "config": {"workload": cfg.name + "_append", "batch": cfg.batch,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
                   "rows": cfg.batch * cfg.n_kv_heads, "fresh_pages": fresh, "replicas": reps,
                   "bytes_per_launch": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "append_kernel", "launches_per_step": 1,
                     "avg_launch_us": round(ms_per_step * 1e3, 3)},
        "cpu_baseline": baseline,
    }
    print(json.dumps(record), flush=True)


def bench_step(args, cfg, lib, torch, np, binding, generate):
    """Time a whole decode step: decode_attn_append writes every sequence's new K/V row at
    position L_b (a fresh page where the token starts one), then decode_attn attends over
    the grown caches (L_b + 1 tokens), with the library's own plan. Two launches per step;
    the pools rotate over replicas as for the attention alone."""
    from decode_phase_attention_paged_amd.workload import ELEM_BYTES, SCALE_BYTES, kv_read_bytes
    log(f"generating {cfg.name} for a decode step ...")
    w = generate(cfg)
    table, positions, fresh = grow_for_append(w, np, cfg)
    lens = (positions + 1).astype(np.int32)
    n_pages = w.num_pages + fresh
    grow = lambda a: None if a is None else np.concatenate(
        [a, np.zeros((fresh,) + a.shape[1:], dtype=a.dtype)])
    k_host, v_host, ks_host, vs_host = (grow(a) for a in (w.k_pages, w.v_pages, w.k_scale,
                                                          w.v_scale))
    rng = np.random.default_rng(w.seed + 1)
    shape = (cfg.batch, cfg.n_kv_heads, cfg.head_dim)
    new = [rng.standard_normal(shape, dtype=np.float32) for _ in range(2)]
    new = [(x.view(np.uint32) >> 16).astype(np.uint16) if cfg.kv_dtype == "bf16"
           else x.astype(np.float16) for x in new]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: device_tensor(torch, np, a, dev)
    q, bt, pos, sl, kn, vn = (t(a) for a in (w.q, table, positions, lens, new[0], new[1]))
    pool_bytes = 2 * k_host.nbytes + (2 * ks_host.nbytes if ks_host is not None else 0)
    reps = replicas_for(args, pool_bytes)
    pools = [(t(k_host), t(v_host), t(ks_host), t(vs_host)) for _ in range(reps)]
    out = torch.empty(w.q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s_handle = ctypes.c_void_p(stream.cuda_stream)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    kv_type = binding._KV_CODES[cfg.kv_dtype]
    append_args, attn_args = [], []
    for kp, vp, ks, vs in pools:
        append_args.append((p(kn), p(vn), p(bt), p(pos), cfg.batch, cfg.max_blocks_per_seq,
                            n_pages, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, kv_type,
                            p(kp), p(vp), p(ks), p(vs), s_handle))
        attn_args.append((p(q), p(kp), p(vp), p(ks), p(vs), p(bt), p(sl), cfg.batch,
                          cfg.max_blocks_per_seq, n_pages, cfg.n_q_heads, cfg.n_kv_heads,
                          cfg.head_dim, cfg.block_size, kv_type, float(w.scale), p(out),
                          s_handle))

    def step(i):
        st = lib.decode_attn_append(*append_args[i % reps])
        if st == 0:
            st = lib.decode_attn(*attn_args[i % reps])
        if st != 0:
            raise RuntimeError(f"decode step failed: {binding.STATUS.get(st, st)}")

    kv_bytes = kv_read_bytes(lens, cfg.n_kv_heads, cfg.head_dim, ELEM_BYTES[cfg.kv_dtype],
                             SCALE_BYTES[cfg.kv_dtype])
    nbytes = kv_bytes + append_bytes(cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.kv_dtype)
    log(f"step: fresh_pages={fresh} replicas={reps} bytes/step={nbytes}")
    ms_per_step, st = timed_record(args, torch, stream, step, nbytes)
    gbs = nbytes / (ms_per_step / 1e3) / 1e9
    log(f"us/step median {ms_per_step * 1e3:.2f} GB/s={gbs:.1f}")
    record = {
        "metric": "decode step (K/V append + attention) GB/s (fraction of MI355X HBM peak) + µs/step",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": getattr(args, "warmup_run", args.warmup),
        "repeats": args.repeats,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_min_max": [round(st["min_ms"] * 1e3, 3), round(st["max_ms"] * 1e3, 3)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
        "argv": sys.argv[1:],
        "config": {"workload": cfg.name + "_step", "batch": cfg.batch,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "kv_dtype": cfg.kv_dtype, "fresh_pages": fresh, "replicas": reps,
                   "bytes_per_step": int(nbytes)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "append_kernel + attention", "launches_per_step": None,
                     "avg_launch_us": None, "step_us": round(ms_per_step * 1e3, 3)},
        "cpu_baseline": None,
    }
    print(json.dumps(record), flush=True)


def prefill_cpu_baseline(w, q, q_start, budget_s: float = 10.0):
    """oracle.prefill_attention as it stands, timed on the host over whole sequences."""
    import numpy as np
    import oracle
    from decode_phase_attention_paged_amd.workload import prefill_flops
    c = w.config
    cores, model = host_info()
    done_flops, spent, seqs = 0, 0.0, 0
    order = np.argsort(w.seq_lens)
    with _ThreadLimit(cores):
        for b in order:
            rows = slice(int(q_start[b]), int(q_start[b + 1]))
            sub = np.array([0, q_start[b + 1] - q_start[b]], dtype=np.int32)
            t0 = time.perf_counter()
            oracle.prefill_attention(q[rows], w.k_pages, w.v_pages, w.block_table[b:b + 1],
                                     w.seq_lens[b:b + 1], sub, w.scale, w.k_scale, w.v_scale)
            spent += time.perf_counter() - t0
            done_flops += prefill_flops(w.seq_lens[b:b + 1], sub, c.n_q_heads, c.head_dim)
            seqs += 1
            if spent >= budget_s:
                break
    return {"value": round(done_flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{seqs} of {c.batch} sequences, shortest first ({spent:.1f} s)"}


def bench_prefill(args, cfg, lib, torch, np, binding, generate):
    """Time decode_attn_prefill: every sequence's last C_b = min(chunk, L_b) tokens attend
    causally over its cache, all sequences in one launch. Throughput counts the algorithmic
    flops (4 D per visible token per row and query head)."""
    from decode_phase_attention_paged_amd.workload import prefill_flops, prefill_rows
    if cfg.chunk <= 0:
        raise SystemExit(f"preset {cfg.name} has no chunk size; use a prefill preset")
    log(f"generating {cfg.name} ...")
    if args.kv and args.kv != cfg.kv_dtype:
        cfg = cfg.with_(kv_dtype=args.kv, name=f"{cfg.name}_{args.kv}")
    w = generate(cfg)
    q_host, qs_host = prefill_rows(w)
    flops = prefill_flops(w.seq_lens, qs_host, cfg.n_q_heads, cfg.head_dim)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: device_tensor(torch, np, a, dev)
    q, qs, bt, sl = t(q_host), t(qs_host), t(w.block_table), t(w.seq_lens)
    pool_bytes = 2 * w.k_pages.nbytes
    reps = replicas_for(args, pool_bytes)
    pools = [(t(w.k_pages), t(w.v_pages)) for _ in range(reps)]
    ks, vs = t(w.k_scale), t(w.v_scale)
    out = torch.empty(q_host.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s_handle = ctypes.c_void_p(stream.cuda_stream)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    total = q_host.shape[0]
    pz = lambda x: None if x is None else p(x)
    kv = {"fp16": binding.KV_FP16, "bf16": binding.KV_BF16, "int8": binding.KV_INT8,
          "fp8": binding.KV_FP8}[cfg.kv_dtype]
    call_args = [(p(q), p(qs), p(kp), p(vp), pz(ks), pz(vs), p(bt), p(sl), cfg.batch, total,
                  cfg.max_blocks_per_seq, w.num_pages, cfg.n_q_heads, cfg.n_kv_heads,
                  cfg.head_dim, cfg.block_size, kv, cfg.chunk, float(w.scale),
                  p(out), s_handle) for kp, vp in pools]

    def step(i):
        st = lib.decode_attn_prefill(*call_args[i % reps])
        if st != 0:
            raise RuntimeError(f"decode_attn_prefill failed: {binding.STATUS.get(st, st)}")

    log(f"prefill: rows={total} chunk={cfg.chunk} replicas={reps} flops/step={flops / 1e9:.1f} G")
    ms_per_step, st = timed_record(args, torch, stream, step, flops)
    tflops = flops / (ms_per_step / 1e3) / 1e12
    log(f"us/launch median {ms_per_step * 1e3:.2f} TFLOP/s={tflops:.1f} "
        f"({tflops / MFMA_F16_PEAK_TFLOPS:.3f} of peak)")
    prof, prof_src = read_profile(cfg.name, "prefill")
    traffic = profile_traffic(prof) if prof else None
    log(f"profile: {prof_src}")
    baseline = None
    if not args.no_cpu_baseline:
        baseline = prefill_cpu_baseline(w, q_host, qs_host)
        log(f"cpu baseline: {baseline}")
    record = {
        "metric": "chunked-prefill attention TFLOP/s (fraction of MI355X fp16 matrix peak)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": getattr(args, "warmup_run", args.warmup),
        "repeats": args.repeats,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_min_max": [round(st["min_ms"] * 1e3, 3), round(st["max_ms"] * 1e3, 3)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
        "argv": sys.argv[1:],
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype, "chunk": cfg.chunk,
                   "rows": total,
                   "seq_lens": f"uniform [{cfg.len_lo}, {cfg.len_hi}], seed {w.seed}",
                   "flops_per_step": int(flops), "kv_bytes_per_step": int(w.kv_bytes),
                   "replicas": reps},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_kernel", "launches_per_step": 1,
                     "avg_launch_us": round(ms_per_step * 1e3, 3)},
        "cpu_baseline": baseline,
    }
    print(json.dumps(record), flush=True)


def decode_step_tiles(cfg, np):
    """The (page, KV head) tiles one decode step of the workload reads, as tile indices
    page * n_kv_heads + head in the order of the sequences and heads, and the number of
    tiles in its pool."""
    from decode_phase_attention_paged_amd.workload import layout
    lens, table, num_pages = layout(cfg)
    hkv = cfg.n_kv_heads
    nb = -(-lens.astype(np.int64) // cfg.block_size)
    parts = [table[b, :nb[b]].astype(np.int64) * hkv + g
             for b in range(cfg.batch) for g in range(hkv)]
    tiles = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return tiles.astype(np.int32), num_pages * hkv


def bench_hbm(args, cfg, torch, np, binding):
    """Reference read rates for the HBM roofline (decode_attn_hbm_reference): a random
    gather of the K and V tiles of one decode step of the workload (every (sequence, KV
    head, page) tile the step reads, in full, in the order of the sequences and heads:
    4 KiB tiles for 16-bit formats, 2 KiB of codes plus the 64-byte row-scale records for
    INT8 and FP8), and a plain streaming read of 4 GiB, over several launch shapes. The
    pools rotate over replicas of at least 1 GiB in all, as in the decode bench, so the
    Infinity Cache cannot serve them. Prints one JSON line; `best_gather_gbs` is the
    attainable rate the decode kernels' roofline fraction can be read against."""
    elem = 2 if cfg.kv_dtype in ("fp16", "bf16") else 1
    tile_bytes = cfg.head_dim * cfg.block_size * elem
    if cfg.head_dim != 128 or cfg.block_size != 16:
        raise SystemExit("the reference gather reads the tiles of head_dim 128, 16-token pages")
    kind = binding.HBM_GATHER if elem == 2 else binding.HBM_GATHER_SCALED
    tiles, pool_tiles = decode_step_tiles(cfg, np)
    count = int(tiles.size)
    scale_bytes = 64 if elem == 1 else 0
    pool_bytes = 2 * pool_tiles * (tile_bytes + scale_bytes)
    reps = replicas_for(args, pool_bytes)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = torch.zeros(reps * pool_tiles * tile_bytes, dtype=torch.uint8, device=dev)
    v = torch.zeros_like(k)
    ks = vs = None
    if scale_bytes:
        ks = torch.zeros(reps * pool_tiles * scale_bytes, dtype=torch.uint8, device=dev)
        vs = torch.zeros_like(ks)
    tile_lists = [torch.from_numpy(tiles + r * pool_tiles).to(dev) for r in range(reps)]
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(65535 * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    gather_bytes = 2 * count * (tile_bytes + scale_bytes)
    results = {"gather": [], "stream": []}

    def measure(kind, depth, nt, grid):
        if kind != binding.HBM_STREAM:
            step = lambda i: binding.hbm_reference(kind, k, sink, b=v, tiles=tile_lists[i % reps],
                                                   a_scale=ks, b_scale=vs, depth=depth,
                                                   nontemporal=nt, grid=grid)
            nbytes = gather_bytes
        else:
            step = lambda i: binding.hbm_reference(kind, buf, sink, depth=depth,
                                                   nontemporal=nt, grid=grid)
            nbytes = buf.numel()
        ms, st = timed_record(args, torch, stream, step, nbytes)
        row = {"depth": depth, "nontemporal": bool(nt), "grid": grid,
               "us_per_launch": round(ms * 1e3, 3),
               "gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
               "gbs_min_max": [round(nbytes / (st["max_ms"] / 1e3) / 1e9, 1),
                               round(nbytes / (st["min_ms"] / 1e3) / 1e9, 1)]}
        log(f"{'stream' if kind == binding.HBM_STREAM else 'gather'} {row}")
        return row

    for nt in (1, 0):
        for depth in (1, 2, 4):
            for grid in (256, 512, 1024, 2048):
                results["gather"].append(measure(kind, depth, nt, grid))
        for depth in (8, 16):
            for grid in (512, 1024, 2048):
                results["stream"].append(measure(binding.HBM_STREAM, depth, nt, grid))
    if int(sink.abs().sum().item()) != 0:
        raise RuntimeError("the reference reads folded to their sink key on zero-filled memory")
    best = {key: max(r["gbs"] for r in rows) for key, rows in results.items()}
    record = {
        "metric": "HBM reference read rate (random K/V tile gather; streaming read)",
        "unit": "GB/s",
        "best_gather_gbs": best["gather"],
        "best_stream_gbs": best["stream"],
        "peak_gbs": HBM_PEAK_GBS,
        "best_gather_frac_of_peak": round(best["gather"] / HBM_PEAK_GBS, 4),
        "best_stream_frac_of_peak": round(best["stream"] / HBM_PEAK_GBS, 4),
        "steps": args.steps,
        "repeats": args.repeats,
        "argv": sys.argv[1:],
        "config": {"workload": cfg.name, "kv_dtype": cfg.kv_dtype, "tile_bytes": tile_bytes,
                   "scale_record_bytes": scale_bytes, "tile_pairs_per_launch": count,
                   "gather_bytes_per_launch": gather_bytes, "pool_tiles": pool_tiles,
                   "replicas": reps, "stream_bytes_per_launch": buf.numel()},
        "gather": results["gather"],
        "stream": results["stream"],
    }
    print(json.dumps(record), flush=True)


# ---------------------------------------------------------------------------------------
# Profile summaries. Layout of DIR for one workload tagged TAG (each a rocprofv3 output
# directory written with `-d DIR/<name> -o run --output-format csv`, next to the bench.py
# JSON line the profiled run printed, DIR/<name>.json):
#   trace_TAG               --kernel-trace --stats
#   pmc_FETCH_SIZE_TAG      --pmc FETCH_SIZE
#   pmc_WRITE_SIZE_TAG      --pmc WRITE_SIZE
#   pmc_FETCH_SIZE_copy, pmc_WRITE_SIZE_copy   the same counters over bench.py --copy-calibration
#   pmc_<P>_TAG             optional further counter passes (any name P), e.g. the SQ and
#                           TCC/TCP sets below
COUNTER_PASSES = {
    "sq_a": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY",
             "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU",
             "GRBM_GUI_ACTIVE"],
    "sq_b": ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_INSTS_SMEM",
             "SQ_ACTIVE_INST_VMEM", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_VMEM",
             "GRBM_GUI_ACTIVE"],   # SQ_ACTIVE_INST_VMEM reads 0 on gfx950
    "mem": ["TCC_HIT_sum", "TCC_MISS_sum", "TCP_UTCL1_TRANSLATION_MISS_sum",
            "TCP_UTCL1_TRANSLATION_HIT_sum", "TCP_TCC_READ_REQ_sum"],
    # L2-to-memory read requests by size: FETCH_SIZE's expression counts a 128-byte request
    # as 64 bytes on gfx950 (hence the copy calibration); these give the bytes directly.
    "rdreq": ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
              "TCC_EA0_RDREQ_sum"],
}


def _csv_rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _last_json(path):
    with open(path) as f:
        lines = [ln for ln in f.read().strip().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def _pmc(dirpath):
    """{kernel: {counter: [value per dispatch]}} of one --pmc output directory."""
    by = {}
    for r in _csv_rows(os.path.join(dirpath, "run_counter_collection.csv")):
        by.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    return by


def _mean(v):
    return sum(v) / len(v) if v else 0.0


def summarize_hbm(d: str, tag: str, rec):
    """profiles/hbm_reference_<workload>.txt: the reference read rates of one
    `bench.py --op hbm` run under rocprofv3 --kernel-trace --stats, with the trace's
    average duration of each (kernel, grid) next to the event-timed figures."""
    argv = [a for a in rec.get("argv", []) if a]
    workload = rec["config"]["workload"]
    by = {}
    for r in _csv_rows(os.path.join(d, f"trace_{tag}", "run_kernel_trace.csv")):
        name = r["Kernel_Name"]
        if "ref_gather_kernel" not in name and "ref_stream_kernel" not in name:
            continue
        short = name.split("::")[-1].split("(")[0]      # ref_gather_kernel<2, true>
        key = (short, int(r["Grid_Size_X"]) // 256)
        by.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    cmd = "python3 $REPO/bench.py " + " ".join(argv)
    out = [f"# rocprofv3 summary: HBM reference reads, workload {workload}",
           f"# {json.dumps(rec['config'])}",
           "# $REPO is the repository root; the command runs from /tmp with TMPDIR=/tmp.",
           f"# summarised by: python3 $REPO/bench.py --summarize-profile $REPO/gpurun_out/prof --tag {tag}",
           f"command_trace: rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof/trace_{tag} -o run -- {cmd}",
           f"kernel_source_sha256: {kernel_source_hash(HBM_SOURCES)}",
           "",
           "## kernel trace (per (kernel, grid): every launch of the run, warm-up included)"]
    for (name, grid), ns in sorted(by.items()):
        out.append(f"{name} grid {grid}: calls {len(ns)}  avg_ns {_mean(ns):.1f}  "
                   f"median_ns {statistics.median(ns):.0f}")
    out += ["", "## event-timed rates (median window; bytes per launch over its time)",
            f"gather bytes per launch: {rec['config']['gather_bytes_per_launch']} "
            f"({rec['config']['tile_pairs_per_launch']} K/V tile pairs of "
            f"{rec['config'].get('tile_bytes', 4096)} bytes"
            + (f" and their {rec['config']['scale_record_bytes']}-byte scale records)"
               if rec['config'].get('scale_record_bytes') else ")"),
            f"stream bytes per launch: {rec['config']['stream_bytes_per_launch']}"]
    for kind in ("gather", "stream"):
        for r in rec[kind]:
            out.append(f"{kind} depth {r['depth']} nontemporal {int(r['nontemporal'])} grid "
                       f"{r['grid']}: {r['us_per_launch']} us  {r['gbs']} GB/s  "
                       f"(windows {r['gbs_min_max'][0]}-{r['gbs_min_max'][1]})")
    out += ["", "## figures used in the roofline discussion",
            f"best_gather_gbs: {rec['best_gather_gbs']}",
            f"best_gather_frac_of_peak: {rec['best_gather_frac_of_peak']}",
            f"best_stream_gbs: {rec['best_stream_gbs']}",
            f"best_stream_frac_of_peak: {rec['best_stream_frac_of_peak']}"]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"hbm_reference_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}: best gather {rec['best_gather_gbs']} GB/s, "
          f"best stream {rec['best_stream_gbs']} GB/s")


def summarize_profile(d: str, tag: str):
    d = os.path.abspath(d)
    trace_dir = os.path.join(d, f"trace_{tag}")
    rec = _last_json(os.path.join(d, f"trace_{tag}.json"))
    argv = [a for a in rec.get("argv", []) if a]
    if "--op" in argv and argv[argv.index("--op") + 1] == "hbm":
        return summarize_hbm(d, tag, rec)
    op = "attn"
    if "--op" in argv:
        op = argv[argv.index("--op") + 1]
    elif "prefill" in rec["metric"]:
        op = "prefill"
    elif "append" in rec["metric"]:
        op = "append" if rec["metric"].startswith("decode K/V append") else "step"
    workload = rec["config"]["workload"]
    for suffix in ("_append", "_step"):
        if op != "attn" and workload.endswith(suffix):
            workload = workload[: -len(suffix)]
    prefix = PREFIX_OF_OP[op]
    timed = rec["steps"] * rec.get("repeats", 1)

    rows = _csv_rows(os.path.join(trace_dir, "run_kernel_trace.csv"))
    by, res = {}, {}
    for r in rows:
        name = r["Kernel_Name"]
        if name.startswith("__amd") or "elementwise" in name or "Memcpy" in name:
            continue
        by.setdefault(name, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        res[name] = (r.get("VGPR_Count"), r.get("Accum_VGPR_Count"), r.get("SGPR_Count"),
                     r.get("LDS_Block_Size"), r.get("Scratch_Size"), r.get("Grid_Size_X"),
                     r.get("Workgroup_Size_X"))
    # The counter passes of this tag only: pmc_<pass>_<tag> for the known pass names (a
    # suffix match would also take, say, pmc_FETCH_SIZE_append_cfg2 for tag cfg2).
    passes = {}
    for pname in ["FETCH_SIZE", "WRITE_SIZE", *COUNTER_PASSES]:
        full = os.path.join(d, f"pmc_{pname}_{tag}")
        if os.path.isdir(full):
            passes[pname] = _pmc(full)

    def counters_of(kernel):
        merged = {}
        for pname, pk in passes.items():
            for cname, vals in pk.get(kernel, {}).items():
                merged.setdefault(cname, vals)
        return merged

    cf, cw = _pmc(os.path.join(d, "pmc_FETCH_SIZE_copy")), _pmc(os.path.join(d, "pmc_WRITE_SIZE_copy"))
    fmax = max(max(v.get("FETCH_SIZE", [0.0])) for v in cf.values())
    wmax = max(max(v.get("WRITE_SIZE", [0.0])) for v in cw.values())
    fetch_scale = (1 << 30) / 1024 / fmax
    write_scale = (1 << 30) / 1024 / wmax

    base_cmd = "python3 $REPO/bench.py " + " ".join(
        a for a in argv)
    out = [f"# rocprofv3 summary: {prefix}, workload {workload}",
           f"# {json.dumps(rec['config'])}",
           "# $REPO is the repository root; each command runs from /tmp with TMPDIR=/tmp.",
           f"# summarised by: python3 $REPO/bench.py --summarize-profile $REPO/gpurun_out/prof --tag {tag}",
           f"command_trace: rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof/trace_{tag} -o run -- {base_cmd}"]
    for pname, pk in passes.items():
        names = sorted({c for k in pk.values() for c in k})
        pj = os.path.join(d, f"pmc_{pname}_{tag}.json")
        pargv = " ".join(_last_json(pj).get("argv", [])) if os.path.exists(pj) else " ".join(argv)
        out.append(f"command_pmc_{pname}: rocprofv3 --pmc {' '.join(names)} --output-format csv "
                   f"-d $REPO/gpurun_out/prof/pmc_{pname}_{tag} -o run -- python3 $REPO/bench.py {pargv}")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        out.append(f"command_copy_{c.split('_')[0].lower()}: rocprofv3 --pmc {c} --output-format csv "
                   f"-d $REPO/gpurun_out/prof/pmc_{c}_copy -o run -- python3 $REPO/bench.py --copy-calibration")
    out.append(f"kernel_source_sha256: {kernel_source_hash(SOURCES_OF_OP[op])}")
    out.append("")
    out.append(f"## kernel trace (per launch; \"timed\" = the last {timed} launches of each kernel, "
               f"the ones bench.py times)")
    dom, dom_total, stats = None, -1, {}
    for k, v in by.items():
        tv = v[-timed:]
        avg, tavg = _mean(v), _mean(tv)
        ctr = counters_of(k)
        stats[k] = (avg, tavg, ctr)
        vg, ag, sg, lds, scr, grid, wg = res[k]
        out.append(f"kernel: {k}")
        out.append(f"  calls {len(v)}  avg_ns {avg:.1f}  timed_avg_ns {tavg:.1f}  min_ns {min(v)}  "
                   f"max_ns {max(v)}  median_ns {statistics.median(v):.0f}")
        out.append(f"  resources: vgpr {vg} agpr {ag} sgpr {sg} lds_bytes {lds} scratch_bytes {scr} "
                   f"grid_threads {grid} workgroup {wg}")
        for cname in sorted(ctr):
            out.append(f"  {cname}_per_dispatch {_mean(ctr[cname]):.2f}")
        if sum(v) > dom_total:
            dom, dom_total = k, sum(v)
    out.append("")
    out.append("## copy calibration (torch copy of 1 GiB: reads 1 GiB, writes 1 GiB)")
    out.append(f"copy_fetch_kib_per_dispatch: {fmax:.2f}")
    out.append(f"copy_write_kib_per_dispatch: {wmax:.2f}")
    out.append(f"fetch_scale: {fetch_scale:.4f}")
    out.append(f"write_scale: {write_scale:.4f}")
    out.append("")
    avg, tavg, ctr = stats[dom]
    fa, wa = _mean(ctr.get("FETCH_SIZE", [])), _mean(ctr.get("WRITE_SIZE", []))
    traffic = (fa * fetch_scale + wa * write_scale) * 1024
    cfg = rec["config"]
    out.append("## figures used by bench.py (dominant kernel)")
    out.append(f"dominant_kernel: {dom}")
    out.append(f"dominant_kernel_avg_ns: {avg:.1f}")
    out.append(f"dominant_kernel_timed_avg_ns: {tavg:.1f}")
    out.append(f"bench_us_per_step_in_this_run: {rec['us_per_step']}")
    if op == "prefill":
        kv = cfg["kv_bytes_per_step"]
        qo = cfg["rows"] * cfg["n_q_heads"] * cfg["head_dim"] * (2 + 4)   # q 16-bit, out fp32
        alg = kv + qo
        out.append(f"algorithmic_flops_per_launch: {cfg['flops_per_step']}")
        out.append(f"algorithmic_bytes_per_launch: {alg}  (K/V {kv} + q 16-bit and out fp32 {qo})")
        out.append(f"traffic_bytes_per_launch: {traffic:.0f}")
        out.append(f"traffic_over_algorithmic: {traffic / alg:.4f}")
        out.append(f"achieved_tflops_at_trace_timed_avg: {cfg['flops_per_step'] / tavg / 1e3:.1f}")
    else:
        alg = cfg.get("kv_bytes_per_step", cfg.get("bytes_per_launch"))
        out.append(f"algorithmic_bytes_per_launch: {alg}")
        out.append(f"traffic_bytes_per_launch: {traffic:.0f}")
        out.append(f"traffic_over_algorithmic: {traffic / alg:.4f}")
        if op == "attn" and "kv_bytes_per_step" in cfg:
            # The K/V reads are the throughput figure's bytes; the step also reads q (16-bit)
            # and writes out (fp32), which the traffic counters see.
            qo = cfg["batch"] * cfg["n_q_heads"] * cfg["head_dim"] * (2 + 4)
            out.append(f"traffic_over_kv_plus_q_and_out: {traffic / (alg + qo):.4f}  "
                       f"(q 16-bit and out fp32: {qo} bytes)")
        out.append(f"achieved_gbs_at_trace_timed_avg: {alg / tavg:.1f}")
        out.append(f"frac_of_hbm_peak_at_trace_timed_avg: {alg / tavg / HBM_PEAK_GBS:.4f}")
    rd = read_bytes_by_request_size(ctr)
    if rd is not None:
        wb = wa * write_scale * 1024
        out.append(f"read_bytes_by_request_size_per_launch: {rd:.0f}")
        out.append(f"read_plus_write_bytes_over_algorithmic: {(rd + wb) / alg:.4f}  "
                   f"(cross-check of traffic_over_algorithmic without the copy calibration)")
    derived = derived_counters(ctr, tavg)
    if derived:
        out.append("")
        out.append("## derived from the counter passes (dominant kernel, per dispatch)")
        for k, v in derived:
            out.append(f"{k}: {v}")
    path = os.path.join(PROFILES, f"{prefix}_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}: {dom[:70]} timed avg {tavg / 1e3:.2f} us, "
          f"traffic/alg {traffic / alg:.4f}")


# MI355X: 256 compute units of 4 SIMDs in 8 XCDs; SQ cycle counters count quad-cycles.
N_CU, N_SIMD, N_XCD, CLOCK_GHZ = 256, 1024, 8, 2.4


def read_bytes_by_request_size(ctr):
    """Bytes the L2 read from memory for one dispatch, from the request-size counters
    (32, 64 and 128 bytes), or None where they were not collected."""
    names = ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
    if not all(n in ctr for n in names):
        return None
    return sum(size * _mean(ctr[n]) for size, n in zip((32, 64, 128), names))


def derived_counters(ctr, kernel_ns):
    """Readable figures from the raw counters of one kernel, where they were collected.
    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's busy cycles are a eighth of it;
    SQ_WAVE_CYCLES, SQ_WAIT_*, SQ_ACTIVE_* count quad-cycles summed over all waves."""
    m = {k: _mean(v) for k, v in ctr.items()}
    out = []
    gui = m.get("GRBM_GUI_ACTIVE")
    if gui:
        cycles = gui / N_XCD
        out.append(("gpu_busy_cycles_of_the_profiled_dispatch", f"{cycles:.0f}"))
        if "SQ_WAVE_CYCLES" in m:
            out.append(("mean_resident_waves_per_cu",
                        f"{4 * m['SQ_WAVE_CYCLES'] / (cycles * N_CU):.2f}"))
        if "SQ_ACTIVE_INST_VALU" in m:
            out.append(("valu_busy_fraction_per_simd",
                        f"{4 * m['SQ_ACTIVE_INST_VALU'] / (cycles * N_SIMD):.3f}"))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            out.append(("mfma_busy_fraction_per_simd",
                        f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * N_SIMD):.3f}"))
    if m.get("SQ_WAVE_CYCLES"):
        for k in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY"):
            if k in m:
                out.append((k.lower() + "_over_wave_cycles", f"{m[k] / m['SQ_WAVE_CYCLES']:.3f}"))
    if m.get("SQ_WAVES"):
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU", "SQ_INSTS_SMEM",
                  "SQ_INSTS_LDS", "SQ_INSTS_MFMA"):
            if k in m:
                out.append((k.lower() + "_per_wave", f"{m[k] / m['SQ_WAVES']:.1f}"))
    if m.get("TCC_EA0_RDREQ_sum"):
        out.append(("share_of_128_byte_read_requests",
                    f"{m.get('TCC_EA0_RDREQ_128B_sum', 0.0) / m['TCC_EA0_RDREQ_sum']:.4f}"))
    if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m and m["TCC_HIT_sum"] + m["TCC_MISS_sum"] > 0:
        out.append(("l2_hit_fraction", f"{m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.3f}"))
    if "TCP_UTCL1_TRANSLATION_MISS_sum" in m and "TCP_UTCL1_TRANSLATION_HIT_sum" in m:
        tot = m["TCP_UTCL1_TRANSLATION_MISS_sum"] + m["TCP_UTCL1_TRANSLATION_HIT_sum"]
        if tot > 0:
            out.append(("utcl1_translation_miss_fraction",
                        f"{m['TCP_UTCL1_TRANSLATION_MISS_sum'] / tot:.4f}"))
    return out


if __name__ == "__main__":
    main()
