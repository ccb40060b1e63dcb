#!/usr/bin/env python3
"""Decode-phase paged attention on one MI355X: KV-read GB/s and us/step.

One step is one decode_attn call over the whole batch (the streaming kernel and
the merge of the (sequence, head) pairs it cut): one layer's decode attention. The default workload is the Llama-2-7B-shaped MHA batch (batch 48,
32 query = 32 KV heads, head_dim 128, seq_lens uniform in [18, 563], 16-token
pages in a shuffled pool, fp16 K/V ~ N(0, 1)); --config picks another preset.

Inputs are resident in HBM before timing starts. To keep the 256 MB Infinity
Cache from serving the KV reads, the step rotates over R replicas of the page
pools totalling at least 1 GiB. Throughput counts algorithmic KV bytes only:
sum_b L_b * Hkv * 2 * D * elem (plus the fp32 row scales for INT8).

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published peak
METRIC = "decode-attn KV-read GB/s (fraction of MI355X HBM peak) + µs/step"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ATTN_SOURCES = ("api.cpp", "kernels.h", "kernels.hip")
APPEND_SOURCES = ("api.cpp", "kernels.h", "append.hip")
PREFILL_SOURCES = ("api.cpp", "kernels.h", "prefill.hip")
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak, published


def kernel_source_hash(sources=ATTN_SOURCES) -> str:
    """Hash of the sources that decide what a kernel does (the kernel file, the internal
    interface and the host side that plans and launches it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_phase_attention_paged_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str, prefix: str = "decode_attn", sources=ATTN_SOURCES):
    """HBM bytes per launch of the dominant kernel, from the committed rocprofv3 summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the counter reads for a
    plain copy of known size), or None when there is none or the kernels changed since."""
    path = os.path.join(PROFILES, f"{prefix}_{workload_name}.txt")
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
    if fields.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None, "kernel changed since the counters were taken"
    try:
        return float(fields["traffic_bytes_per_launch"]), path
    except (KeyError, ValueError):
        return None, "summary lacks traffic_bytes_per_launch"


def cpu_baseline(w, budget_s: float = 10.0):
    """The fp64 oracle as it stands, timed on the host over a bounded sample."""
    import numpy as np
    import oracle
    from decode_phase_attention_paged_amd.workload import ELEM_BYTES, SCALE_BYTES, kv_read_bytes
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    c = w.config
    # Sample: a prefix of the batch sized to fit the budget (at least one sequence).
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
        oracle.decode_attention(w.q[:n], w.k_pages, w.v_pages, w.block_table[:n], w.seq_lens[:n],
                                w.scale, w.k_scale, w.v_scale)
        spent += time.perf_counter() - t0
        reps += 1
    gbs = sample_bytes * reps / spent / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {c.batch} sequences x {reps} repetitions "
                      f"({sample_bytes * reps / 1e9:.3f} GB of KV in {spent:.1f} s)",
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


# Kernels one step launches, by plan mode (stream, split, segment).
KERNELS = {0: "stream_kernel + piece_merge_kernel", 1: "split_kernel + split_merge_kernel",
           2: "seg_kernel"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=0, choices=[0, 1, 2, 3, 4, 5, 6, 7, 8],
                    help="workload preset (0 = the op's default: 2 for attn and append, "
                         "8 for prefill)")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="stream mode on this many workgroups, or the grid of segment mode "
                         "with --splits 1 (0 = the library's plan)")
    ap.add_argument("--splits", type=int, default=0,
                    help="1 = segment mode, >1 = split mode with this many partitions "
                         "(0 = the library's plan)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >= 1 GiB")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--graph", type=int, default=0,
                    help="capture this many consecutive steps in one HIP graph and time "
                         "replays of it (the step count is rounded up to a multiple)")
    ap.add_argument("--kv", choices=["fp16", "bf16", "int8", "fp8"], default=None,
                    help="prefill only: run the preset's shapes over another storage format")
    ap.add_argument("--op", choices=["attn", "append", "prefill", "step"], default="attn",
                    help="attn: the decode-attention step (default); append: the K/V append "
                         "that precedes it in a decode step, on the same workload; prefill: "
                         "chunked-prefill attention (default workload: the prefill preset)")
    args = ap.parse_args()

    if args.kv is not None and args.op != "prefill":
        ap.error("--kv applies to --op prefill only; the decode presets fix their formats")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library runs decode attention on a single "
              "MI355X, and multi-GPU sharding is a design note only; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from decode_phase_attention_paged_amd import binding
    from decode_phase_attention_paged_amd.workload import CONFIGS, generate

    if args.copy_calibration:
        copy_calibration(torch)
        return

    lib = binding.load_library()
    if args.config == 0:
        args.config = 8 if args.op == "prefill" else 2
    cfg = CONFIGS[args.config]
    if args.op == "append":
        return bench_append(args, cfg, lib, torch, np, binding, generate)
    if args.op == "prefill":
        return bench_prefill(args, cfg, lib, torch, np, binding, generate)
    if args.op == "step":
        return bench_step(args, cfg, lib, torch, np, binding, generate)
    log(f"generating {cfg.name} ...")
    w = generate(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: device_tensor(torch, np, a, dev)
    q, bt, sl = t(w.q), t(w.block_table), t(w.seq_lens)
    pool_bytes = 2 * w.k_pages.nbytes + (2 * w.k_scale.nbytes if w.k_scale is not None else 0)
    reps = args.replicas or max(2, math.ceil((1 << 30) / pool_bytes))
    reps = min(reps, max(1, (48 << 30) // pool_bytes))
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

    def step(i):
        kind, a = call_args[i % reps]
        st = lib.decode_attn(*a) if kind == "auto" else lib.decode_attn_ex(*a)
        if st != 0:
            raise RuntimeError(f"decode_attn failed: {binding.STATUS.get(st, st)}")

    log(f"plan: {plan} replicas={reps} "
        f"pool={pool_bytes / 1e6:.1f} MB kv_bytes/step={w.kv_bytes / 1e6:.1f} MB")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph > 0:
        # The same calls, recorded on a capture stream, args.graph steps per graph; replays
        # run on torch's current stream, where the events below are recorded.
        cap = torch.cuda.Stream()
        handle = ctypes.c_void_p(cap.cuda_stream)
        captured = [(kind, a[:-1] + (handle,)) for kind, a in call_args]
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.graph):
                kind, a = captured[i % reps]
                st = lib.decode_attn(*a) if kind == "auto" else lib.decode_attn_ex(*a)
                if st != 0:
                    raise RuntimeError(f"decode_attn failed in capture: {binding.STATUS.get(st, st)}")
        torch.cuda.synchronize()
        args.steps = -(-args.steps // args.graph) * args.graph
        graph.replay()
        torch.cuda.synchronize()
        log(f"graph: {args.graph} steps per replay, {args.steps // args.graph} replays timed")

    # Timed region: exactly K back-to-back steps between one pair of HIP events recorded
    # on the launch stream. No event sits between steps: an event record between two
    # launches delays the second one by several microseconds on this GPU.
    start_ev = torch.cuda.Event(enable_timing=True)
    stop_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start_ev.record(stream)
    if graph is not None:
        for _ in range(args.steps // args.graph):
            graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    stop_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start_ev.elapsed_time(stop_ev)
    ms_per_step = total_ms / args.steps
    # A step is the main kernel and the merge launched right behind it; back-to-back
    # launches leave no gap, so the step time is the kernels' summed duration and is taken,
    # conservatively, as the duration of the dominant (main) launch.
    avg_launch_s = ms_per_step / 1e3
    gbs = w.kv_bytes * args.steps / (total_ms / 1e3) / 1e9
    achieved = w.kv_bytes / avg_launch_s / 1e9
    log(f"steps={args.steps} total={total_ms:.3f} ms (wall {wall * 1e3:.1f} ms) "
        f"us/step={ms_per_step * 1e3:.2f} GB/s={gbs:.1f} ({gbs / HBM_PEAK_GBS:.3f} of peak)")
    if wall * 1e3 > 1.5 * total_ms:
        log("warning: host launch rate may be limiting the step rate")

    traffic, traffic_src = read_traffic(cfg.name)
    log(f"traffic: {traffic} ({traffic_src})")
    baseline = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        baseline = cpu_baseline(w)
        log(f"cpu baseline: {baseline}")

    record = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
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
            "kernel": KERNELS[plan.mode] + " (one step)",
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
        },
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
    reps, spent = 0, 0.0
    while reps < 1 or (spent < budget_s and reps < 200):
        t0 = time.perf_counter()
        oracle.append_kv(w.k_pages, w.v_pages, table, positions, new[0], new[1], c.block_size,
                         w.k_scale, w.v_scale)
        spent += time.perf_counter() - t0
        reps += 1
    nbytes = append_bytes(c.batch, c.n_kv_heads, c.head_dim, c.kv_dtype)
    return {"value": round(nbytes * reps / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} whole launches ({c.batch * c.n_kv_heads} rows each) in "
                      f"{spent:.1f} s, pool copies included"}


def bench_append(args, cfg, lib, torch, np, binding, generate):
    """Time decode_attn_append: every sequence of the workload writes its next token
    (position L_b) into its page slot; sequences whose next token starts a new page get a
    fresh page. The new rows are fp16 ~ N(0, 1) scaled per row by U(0.1, 10)."""
    log(f"generating {cfg.name} for the append ...")
    w = generate(cfg)
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
    reps = args.replicas or max(2, math.ceil((1 << 30) / pool_bytes))
    reps = min(reps, max(1, (48 << 30) // pool_bytes))
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start_ev = torch.cuda.Event(enable_timing=True)
    stop_ev = torch.cuda.Event(enable_timing=True)
    start_ev.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop_ev.record(stream)
    torch.cuda.synchronize()
    total_ms = start_ev.elapsed_time(stop_ev)
    ms_per_step = total_ms / args.steps
    gbs = nbytes * args.steps / (total_ms / 1e3) / 1e9
    log(f"steps={args.steps} total={total_ms:.3f} ms us/step={ms_per_step * 1e3:.2f} "
        f"GB/s={gbs:.1f}")
    traffic, traffic_src = read_traffic(cfg.name, prefix="decode_attn_append",
                                       sources=APPEND_SOURCES)
    log(f"traffic: {traffic} ({traffic_src})")
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
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp16": "f16", "bf16": "bf16", "int8": "f16->i8",
                  "fp8": "f16->fp8e4m3"}[cfg.kv_dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name + "_append", "batch": cfg.batch,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
                   "rows": cfg.batch * cfg.n_kv_heads, "fresh_pages": fresh, "replicas": reps,
                   "bytes_per_launch": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "append_kernel", "avg_launch_us": round(ms_per_step * 1e3, 3)},
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
    reps = args.replicas or max(2, math.ceil((1 << 30) / pool_bytes))
    reps = min(reps, max(1, (48 << 30) // pool_bytes))
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start_ev = torch.cuda.Event(enable_timing=True)
    stop_ev = torch.cuda.Event(enable_timing=True)
    start_ev.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop_ev.record(stream)
    torch.cuda.synchronize()
    total_ms = start_ev.elapsed_time(stop_ev)
    ms_per_step = total_ms / args.steps
    gbs = nbytes * args.steps / (total_ms / 1e3) / 1e9
    log(f"steps={args.steps} us/step={ms_per_step * 1e3:.2f} GB/s={gbs:.1f}")
    record = {
        "metric": "decode step (K/V append + attention) GB/s (fraction of MI355X HBM peak) + µs/step",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name + "_step", "batch": cfg.batch,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "kv_dtype": cfg.kv_dtype, "fresh_pages": fresh, "replicas": reps,
                   "bytes_per_step": int(nbytes)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "append_kernel + attention (two launches)",
                     "avg_launch_us": None},
        "cpu_baseline": None,
    }
    print(json.dumps(record), flush=True)

def prefill_cpu_baseline(w, q, q_start, budget_s: float = 10.0):
    """oracle.prefill_attention as it stands, timed on the host over whole sequences."""
    import numpy as np
    import oracle
    from decode_phase_attention_paged_amd.workload import prefill_flops
    c = w.config
    done_flops, spent, seqs = 0, 0.0, 0
    order = np.argsort(w.seq_lens)
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
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    return {"value": round(done_flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
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
    reps = args.replicas or max(2, math.ceil((1 << 30) / pool_bytes))
    reps = min(reps, max(1, (48 << 30) // pool_bytes))
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start_ev = torch.cuda.Event(enable_timing=True)
    stop_ev = torch.cuda.Event(enable_timing=True)
    start_ev.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop_ev.record(stream)
    torch.cuda.synchronize()
    total_ms = start_ev.elapsed_time(stop_ev)
    ms_per_step = total_ms / args.steps
    tflops = flops / (ms_per_step / 1e3) / 1e12
    log(f"steps={args.steps} total={total_ms:.3f} ms us/step={ms_per_step * 1e3:.2f} "
        f"TFLOP/s={tflops:.1f} ({tflops / MFMA_F16_PEAK_TFLOPS:.3f} of peak)")
    traffic, traffic_src = read_traffic(cfg.name, prefix="decode_attn_prefill",
                                        sources=PREFILL_SOURCES)
    log(f"traffic: {traffic} ({traffic_src})")
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
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[cfg.kv_dtype],
        "data": "synthetic",
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
                     "kernel": "prefill_kernel", "avg_launch_us": round(ms_per_step * 1e3, 3)},
        "cpu_baseline": baseline,
    }
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
