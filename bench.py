#!/usr/bin/env python3
"""Benchmark: fused chunked top-K KL loss, forward + backward, on one MI355X.

One step = kd_topk_kl_forward + kd_topk_kl_backward over the whole batch of
N positions (every chunk), with inputs already resident in device memory.
Default workload: the very-long-context head (N = 262144 positions, D = 4096,
V = 131072, K = 100, chunk = 4096, T = 1, fp32 dW accumulator), the largest
of the workloads, synthetic seeded inputs.  The timed steps run without any
per-kernel instrumentation; per-kernel averages come from a separate pass of
--profile-steps steps after them.

Prints one JSON line on stdout; everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused top-K KL fwd+bwd tokens/s and % bf16 MFMA peak; peak HBM GiB"
# MI355X published dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
GEMM_KERNELS = ("logits_fwd", "logits_bwd", "dh", "dw")
GROUP_POSITIONS = 8192  # positions per dW GEMM of the library (whole chunks, at most 8)
DH_ROWS = 4096          # rows per dH GEMM within such a group
WORKLOAD_NAMES = {"tiny": "tiny", "toy": "toy_lm_head", "large_vocab": "large_vocab_head",
                  "long": "long_context", "very_long": "very_long_context"}
# HBM traffic per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, one file
# per workload, with the hash of the sources it was measured on (reported only
# while they are unchanged).
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def traffic_path(workload: str) -> str:
    return os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
KERNEL_SOURCES = ("lm_head_top_amd/csrc/kd_kernels.hip", "lm_head_top_amd/csrc/kd_kernels.h",
                  "lm_head_top_amd/csrc/kd_capi.hip", "lm_head_top_amd/csrc/kd_plan.cpp",
                  "lm_head_top_amd/csrc/kd_plan.h")
# demangled kernel name -> the library's kernel class name
KERNEL_PATTERNS = (("logits_kernel<0>", "logits_fwd"), ("logits_kernel<1>", "logits_bwd"),
                   ("dh_reduce_kernel", "dh_reduce"), ("dh_kernel", "dh"), ("dw_kernel", "dw"),
                   ("teacher_kernel", "teacher"), ("bucket_kernel", "bucket"),
                   ("combine_kernel", "combine"), ("finalize_kernel", "finalize"),
                   ("topk_select_kernel", "topk_select"))
COPY_KERNEL_PATTERN = "neg_kernel"   # torch.neg(fp32): reads and writes the calibration bytes once


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_info():
    """(threads, library description) of numpy's BLAS, from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas = []
    if not blas:
        return len(os.sched_getaffinity(0)), "unknown"
    d = max(blas, key=lambda d: d.get("num_threads", 1))
    lib = f"{d.get('internal_api', '?')} {d.get('version', '')} ({os.path.basename(d.get('filepath', ''))})"
    return int(d.get("num_threads", 1)), lib.strip()


def cpu_baseline(inp, cfg, rows, repeats=3):
    """The fp64 oracle, as it stands, on the first `rows` positions of the
    workload (row-blocked with the workload's chunk), median of `repeats`
    runs.  Its cost per position does not depend on N (each block is an
    independent dense problem against the same W), so the rate of the prefix
    is the whole workload's rate, extrapolated linearly."""
    import numpy as np
    from oracle import kl_oracle as O
    threads, blas = _blas_info()
    rows = min(rows, cfg.N)
    H = inp["H"][:rows]
    idx = inp["idx"][:rows]
    t = inp["t"][:rows]
    block = min(cfg.chunk, rows)
    times = []
    for _ in range(max(repeats, 1)):
        t0 = time.perf_counter()
        out = O.forward_backward_blocked(H, inp["W"], idx, t, cfg.T, block=block)
        times.append(time.perf_counter() - t0)
        assert np.isfinite(out["loss"])
        del out
    times.sort()
    dt = times[len(times) // 2]
    extrap = " extrapolated linearly in N" if rows < cfg.N else ""
    return {"value": round(rows / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {cfg.N} positions of the same workload (fp64 numpy oracle, "
                      f"row-blocked, block={block}), median of {len(times)} runs of "
                      f"{', '.join(f'{x:.1f}' for x in times)} s;{extrap}",
            "cpu_model": _host_cpu_model(), "blas": blas,
            "affinity_cores": len(os.sched_getaffinity(0))}


def code_text(src: str) -> str:
    """C/C++ source without comments and with whitespace collapsed: edits to
    comments do not change the code the counters were taken on (the sources
    hold no comment markers inside string literals)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(read=None) -> str:
    """SHA-256 of the kernel sources' code (comments and layout excluded)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel)) as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(rel.encode() + b"\0" + code_text(text).encode())
    return h.hexdigest()


def _kernel_class(name: str):
    for pat, cls in KERNEL_PATTERNS:
        if pat in name:
            return cls
    return None


def _read_counter(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 csv."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _find_csv(d: str) -> str:
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *counter_collection.csv under {d}")


def _config_doc(cfg, seed) -> dict:
    return {"workload": WORKLOAD_NAMES[cfg.name], "N": cfg.N, "D": cfg.D, "V": cfg.V,
            "K": cfg.K, "chunk": cfg.chunk, "T": cfg.T, "seed": seed}


def write_traffic(fetch_dir, write_dir, copy_mib, command, config):
    """Turn two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch for each kernel class, each counter
    scaled by what it reads for a plain fp32 copy of copy_mib MiB."""
    fetch = _read_counter(_find_csv(fetch_dir), "FETCH_SIZE")
    write = _read_counter(_find_csv(write_dir), "WRITE_SIZE")

    def copy_reading(d, what):
        vals = [v for n, vs in d.items() if COPY_KERNEL_PATTERN in n for v in vs]
        if not vals:
            raise SystemExit(f"no {COPY_KERNEL_PATTERN} dispatch in the {what} pass: "
                             "run bench.py with --copy-calibration-mib")
        return max(vals)

    known_kib = copy_mib * 1024.0
    f_scale = known_kib / copy_reading(fetch, "FETCH_SIZE")
    w_scale = known_kib / copy_reading(write, "WRITE_SIZE")
    kernels = {}
    for d, key in ((fetch, "fetch_kib"), (write, "write_kib")):
        for name, vals in d.items():
            cls = _kernel_class(name)
            if cls is None:
                continue
            e = kernels.setdefault(cls, {})
            e[key + "_raw_per_launch"] = sum(vals) / len(vals)
            e["launches_" + key.split("_")[0]] = len(vals)
    for cls, e in kernels.items():
        fb = e.get("fetch_kib_raw_per_launch", 0.0) * f_scale * 1024.0
        wb = e.get("write_kib_raw_per_launch", 0.0) * w_scale * 1024.0
        e.update(fetch_bytes_per_launch=fb, write_bytes_per_launch=wb, bytes_per_launch=fb + wb)
    doc = {"what": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by "
                   "its reading for a plain fp32 copy of known size",
           "source_sha256": source_hash(), "sources": list(KERNEL_SOURCES),
           "calibration": {"copy_mib": copy_mib, "fetch_scale": f_scale, "write_scale": w_scale},
           "command": command, "config": config, "kernels": kernels}
    out = traffic_path(config["workload"])
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
        f.write("\n")
    log(f"wrote {out}: fetch scale {f_scale:.4f}, write scale {w_scale:.4f}")
    for cls, e in sorted(kernels.items()):
        log(f"  {cls:11s} {e['bytes_per_launch'] / 2**20:10.1f} MiB per launch")


def write_stats(stats_dir, out_path, command, bench_line=None):
    """Short text summary of a rocprofv3 --kernel-trace --stats run (its
    kernel_stats.csv), with the bench line the same run printed."""
    path = None
    for root, _, files in os.walk(stats_dir):
        for fn in files:
            if fn.endswith("kernel_stats.csv"):
                path = os.path.join(root, fn)
    if path is None:
        raise SystemExit(f"no *kernel_stats.csv under {stats_dir}")
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel statistics", "", "Command (from the repository root):", "",
             "    " + command, "",
             "| kernel class | calls | total ms | average ms | min ms | max ms | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        cls = _kernel_class(name) or re.sub(r"\(.*", "", name)[:60]
        lines.append(f"| {cls} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e6:.4f} | {float(r['MinNs']) / 1e6:.4f} | "
                     f"{float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.2f} |")
    if bench_line:
        lines += ["", "The bench line the same run printed:", "", "    " + bench_line.strip()]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {out_path}")


def measured_traffic(kernel: str, config: dict):
    """Bytes per launch of `kernel` if the workload's traffic file was taken on
    the current sources and the same workload, else None."""
    try:
        with open(traffic_path(config["workload"])) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("source_sha256") != source_hash() or doc.get("config") != config:
        return None
    e = doc.get("kernels", {}).get(kernel)
    return None if e is None else e["bytes_per_launch"]


def _gpu_inputs(torch, N, D, V, K, seed, dev):
    """Seeded device-side random inputs of the workload's shapes (for the memory
    sweep, whose largest sizes are slow to draw on the host)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    H = torch.randn((N, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    idx = torch.randint(0, V, (N, K), generator=g, device=dev, dtype=torch.int32)
    t = torch.sort(torch.randn((N, K), generator=g, device=dev) * 3 ** 0.5, dim=1,
                   descending=True).values
    return H, idx, t


def memory_sweep(args):
    """Peak device memory and time of one forward + backward for growing N at
    D = 4096, V = 131072, K = 100, chunk = 2048: the fused loss keeps memory
    linear in N (no N x V term).  Prints one JSON line with the fit."""
    import numpy as np
    import torch
    import lm_head_top_amd as kd
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    D, V, K, chunk, T = 4096, 131072, 100, 2048, 1.0
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    W = (torch.randn((V, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    dW = torch.zeros((V, D), dtype=torch.float32, device=dev)
    points = []
    for N in args.sweep_n:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        H, idx, t = _gpu_inputs(torch, N, D, V, K, args.seed + N, dev)
        loss, lse = kd.forward(H, W, idx, t, T, chunk)  # warm-up call
        kd.backward(H, W, idx, t, lse, None, T, chunk, dW=dW)
        del loss, lse
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        loss, lse = kd.forward(H, W, idx, t, T, chunk)
        dH, _ = kd.backward(H, W, idx, t, lse, None, T, chunk, dW=dW)
        e1.record()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated()
        ms = e0.elapsed_time(e1)
        points.append({"N": N, "peak_gib": round(peak / 2**30, 4), "ms": round(ms, 3),
                       "tokens_per_s": round(N / (ms * 1e-3), 1)})
        log(f"N={N}: peak {peak / 2**30:.3f} GiB, {ms:.2f} ms, loss {loss.item():.5f}")
        del H, idx, t, loss, lse, dH
    x = np.array([p["N"] for p in points], dtype=np.float64)
    y = np.array([p["peak_gib"] for p in points], dtype=np.float64) * 2**30
    slope, icpt = np.polyfit(x, y, 1)
    resid = float(np.max(np.abs(y - (slope * x + icpt)) / y))
    line = {"mode": "memory_sweep", "D": D, "V": V, "K": K, "chunk": chunk,
            "points": points, "slope_kib_per_token": round(slope / 1024, 3),
            "intercept_gib": round(icpt / 2**30, 3), "max_rel_residual": round(resid, 5),
            "note": "peak = torch.cuda.max_memory_allocated over one forward + backward, "
                    "including W, dW, H, cache, lse, dH and the workspace"}
    print(json.dumps(line), flush=True)


def dense_reference(args):
    """The dense loss in plain PyTorch eager autograd (full [N, V] logits in fp32)
    beside the fused loss on the same inputs: peak memory and time of one
    forward + backward.  A measurement aid; the library does not use it."""
    import numpy as np
    import torch
    import lm_head_top_amd as kd
    from synth import get_config, make_inputs
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    if args.dense_n > 0:
        cfg = cfg.replace(N=args.dense_n)
    inp = make_inputs(cfg, args.seed)
    H = torch.from_numpy(inp["H"].view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(inp["idx"]).to(dev)
    t = torch.from_numpy(inp["t"]).to(dev)
    N, T = cfg.N, cfg.T

    def dense_step():
        Hg = H.detach().requires_grad_(True)
        Wt = W.detach().t().contiguous().requires_grad_(True)  # [D, V]; plain 2-D products only
        z = (Hg @ Wt).float() / T
        logq = torch.log_softmax(z, dim=-1)
        lq = logq.gather(1, idx.long())
        logp = torch.log_softmax(t / T, dim=-1)
        loss = (logp.exp() * (logp - lq)).sum() / N
        loss.backward()
        return loss.detach(), Hg.grad, Wt.grad

    def fused_step():
        loss, lse = kd.forward(H, W, idx, t, T, cfg.chunk)
        dH, dW = kd.backward(H, W, idx, t, lse, None, T, cfg.chunk)
        return loss, dH, dW

    out = {}
    for name, fn in (("fused", fused_step), ("dense", dense_step)):
        fn()  # warm-up (library and allocator)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            res = fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        peak = torch.cuda.max_memory_allocated()
        out[name] = {"ms_median": round(sorted(times)[1], 3), "peak_gib": round(peak / 2**30, 3),
                     "peak_above_inputs_gib": round((peak - base) / 2**30, 3),
                     "loss": float(res[0].item())}
        log(f"{name}: {out[name]}")
        del res
    rel = abs(out["fused"]["loss"] - out["dense"]["loss"]) / abs(out["dense"]["loss"])
    line = {"mode": "dense_reference", "config": _config_doc(cfg, args.seed), **out,
            "loss_rel_diff": rel,
            "dense_grid_fp32_gib": round(N * cfg.V * 4 / 2**30, 3),
            "speedup_fused_over_dense": round(out["dense"]["ms_median"] / out["fused"]["ms_median"], 3),
            "memory_ratio_dense_over_fused": round(out["dense"]["peak_gib"] / out["fused"]["peak_gib"], 3)}
    print(json.dumps(line), flush=True)


def topk_writer(args):
    """Teacher top-K cache writer on teacher logits of the workload's shape
    (N x V, fp32 or bf16, drawn on the device from a seeded generator): time
    per call and HBM bandwidth against the 8 TB/s roofline (the logits are read
    once; the cache written is N * K * 8 bytes)."""
    import torch
    import lm_head_top_amd as kd
    from synth import get_config
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    N, V, K = cfg.N, cfg.V, cfg.K
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    x = torch.randn((N, V), generator=g, device=dev) * 3 ** 0.5
    if args.topk_dtype == "bf16":
        x = x.to(torch.bfloat16)
    esz = x.element_size()
    for _ in range(args.warmup):
        kd.topk_select(x, K)
    kd.profile_enable(("topk_select",))
    kd.profile_read("topk_select")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        idx, val = kd.topk_select(x, K)
    e1.record()
    torch.cuda.synchronize()
    kd.profile_enable(None)
    ms, n = kd.profile_read("topk_select")
    avg = ms / max(n, 1)
    bytes_call = N * V * esz + N * K * 8
    gbs = bytes_call / (avg * 1e-3) / 1e9
    line = {"mode": "topk_writer", "metric": "teacher top-K cache writer rows/s", "unit": "rows/s",
            "value": round(N / (e0.elapsed_time(e1) / args.steps * 1e-3), 1),
            "ms_per_call": round(e0.elapsed_time(e1) / args.steps, 4), "steps": args.steps,
            "dtype": args.topk_dtype, "config": {"workload": f"teacher logits of {WORKLOAD_NAMES[cfg.name]}",
                                                 "N": N, "V": V, "K": K, "seed": args.seed},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbs / 8000.0, 4), "traffic": None,
                         "avg_launch_ms": round(avg, 4), "bytes_per_launch": bytes_call}}
    print(json.dumps(line), flush=True)


def keep_compare(args):
    """The fused loss (recomputes each chunk in the backward, 8 N D V flops,
    O(chunk V) memory) beside the comparators that keep instead of
    recomputing, on the same inputs: kept gradient (bf16 G for all N, 6 N D V
    flops) and kept logits (every chunk's fp32 logits, the pages' next-best
    variant, 6 N D V flops).  Each mode runs on its own, with the device
    memory of the previous one released: time of one forward + backward
    (median of --steps) and peak memory.  A measurement aid."""
    import torch
    import lm_head_top_amd as kd
    from synth import get_config
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    N, D, V, K, T, chunk = cfg.N, cfg.D, cfg.V, cfg.K, cfg.T, cfg.chunk
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    W = (torch.randn((V, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    H, idx, t = _gpu_inputs(torch, N, D, V, K, args.seed + 1, dev)
    dW = torch.zeros((V, D), dtype=torch.float32, device=dev)

    def fused():
        loss, lse = kd.forward(H, W, idx, t, T, chunk)
        kd.backward(H, W, idx, t, lse, None, T, chunk, dW=dW)
        return loss

    def keep_grad():
        loss, lse, ws = kd.forward_keep(H, W, idx, t, T, chunk)
        kd.backward_keep(H, W, K, ws, None, T, chunk, dW=dW)
        return loss

    def keep_logits():
        loss, lse, ws = kd.forward_keep_logits(H, W, idx, t, T, chunk)
        kd.backward_keep_logits(H, W, idx, t, lse, ws, None, T, chunk, dW=dW)
        return loss

    modes = {"fused": fused, "kept_gradient": keep_grad, "kept_logits": keep_logits}
    out = {}
    for name in args.keep_modes:
        fn = modes[name]
        fn()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        times = []
        for _ in range(max(args.steps, 1)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            loss = fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        out[name] = {"ms_median": round(times[len(times) // 2], 3),
                     "peak_gib": round(torch.cuda.max_memory_allocated() / 2**30, 3),
                     "loss": float(loss.item())}
        log(f"{name}: {out[name]}")
        del loss
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    line = {"mode": "keep_compare",
            "config": {"workload": WORKLOAD_NAMES[cfg.name], "N": N, "D": D, "V": V, "K": K,
                       "chunk": chunk, "seed": args.seed}, **out,
            "dense_grid_fp32_gib": round(N * V * 4 / 2**30, 3)}
    for name in out:
        if name != "fused" and "fused" in out:
            line[f"time_ratio_{name}_over_fused"] = round(out[name]["ms_median"] / out["fused"]["ms_median"], 3)
            line[f"memory_ratio_{name}_over_fused"] = round(out[name]["peak_gib"] / out["fused"]["peak_gib"], 3)
    print(json.dumps(line), flush=True)


def blas_compare(args):
    """The library's four GEMM kernels beside hipBLASLt (torch.mm) on the same
    shapes of --config: the forward / backward logits GEMM of one chunk
    (H_c W^T), the dH GEMM of one block of a group (G W) and the dW GEMM of
    one group of chunks (G^T H).  The library's
    kernels carry their fused epilogues (online log-sum-exp, gradient, fp32
    accumulation into dW); torch.mm writes bf16 and does nothing else.  A
    measurement aid: per-launch averages over --steps fused steps, and the
    median of 10 torch.mm calls."""
    import torch
    import lm_head_top_amd as kd
    from synth import get_config
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    N, D, V, K, T, chunk = cfg.N, cfg.D, cfg.V, cfg.K, cfg.T, cfg.chunk
    c = min(chunk, N)
    # the library's dH and dW GEMMs run over groups of whole chunks holding at
    # least GROUP_POSITIONS positions (at most 8 chunks), capped by N
    rows_dw = min(N, c * min(8, -(-GROUP_POSITIONS // c)))
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    W = (torch.randn((V, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    H, idx, t = _gpu_inputs(torch, N, D, V, K, args.seed + 1, dev)
    dW = torch.zeros((V, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kd.workspace_size(N, D, V, K, chunk), dtype=torch.uint8, device=dev)

    def step():
        loss, lse = kd.forward(H, W, idx, t, T, chunk, workspace=ws)
        kd.backward(H, W, idx, t, lse, None, T, chunk, dW=dW, workspace=ws)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    kd.profile_enable(GEMM_KERNELS)
    for k in GEMM_KERNELS:
        kd.profile_read(k)
    for _ in range(max(args.steps, 1)):
        step()
    torch.cuda.synchronize()
    kd.profile_enable(None)
    ours = {k: kd.profile_read(k) for k in GEMM_KERNELS}
    Hc = H[:c]
    G = torch.randn((rows_dw, V), generator=g, device=dev).to(torch.bfloat16)
    Hg = H[:rows_dw]
    rows_dh = min(rows_dw, DH_ROWS)
    Gh = G[:rows_dh]
    shapes = {"logits_fwd": (lambda: torch.mm(Hc, W.t()), 2 * c * D * V),
              "logits_bwd": (lambda: torch.mm(Hc, W.t()), 2 * c * D * V),
              "dh": (lambda: torch.mm(Gh, W), 2 * rows_dh * D * V),
              "dw": (lambda: torch.mm(G.t(), Hg), 2 * rows_dw * D * V)}
    out = {}
    for k, (fn, flops) in shapes.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        blas_ms = times[5]
        ms, n = ours[k]
        ours_ms = ms / n
        out[k] = {"ours_ms": round(ours_ms, 4), "ours_tflops": round(flops / ours_ms / 1e9, 1),
                  "hipblaslt_ms": round(blas_ms, 4), "hipblaslt_tflops": round(flops / blas_ms / 1e9, 1),
                  "gflop": round(flops / 1e9, 1)}
        log(f"{k}: {out[k]}")
    line = {"mode": "gemm_vs_hipblaslt", "config": {**_config_doc(cfg, args.seed), "dw_rows": rows_dw,
                                                   "dh_rows": rows_dh},
            "kernels": out}
    print(json.dumps(line), flush=True)


def loss_ext(args):
    """The loss extensions on --config beside the plain loss, same inputs: a
    0/1 position mask (about 10% of positions masked, as padding would), a
    hard label per position (about 5% without one) mixed in with weights
    0.5 / 0.5, and T^2 scaling.  Time of one forward + backward each."""
    import torch
    import lm_head_top_amd as kd
    from synth import get_config
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    N, D, V, K, T, chunk = cfg.N, cfg.D, cfg.V, cfg.K, cfg.T, cfg.chunk
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    W = (torch.randn((V, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    H, idx, t = _gpu_inputs(torch, N, D, V, K, args.seed + 1, dev)
    mask = (torch.rand(N, generator=g, device=dev) >= 0.1).float()
    labels = torch.randint(0, V, (N,), generator=g, device=dev, dtype=torch.int32)
    labels[torch.rand(N, generator=g, device=dev) < 0.05] = -1
    dW = torch.zeros((V, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kd.workspace_size(N, D, V, K, chunk), dtype=torch.uint8, device=dev)
    ext = dict(row_weight=mask, labels=labels, kd_weight=0.5, ce_weight=0.5, scale_T2=True)

    def plain():
        loss, lse = kd.forward(H, W, idx, t, T, chunk, workspace=ws)
        kd.backward(H, W, idx, t, lse, None, T, chunk, dW=dW, workspace=ws)
        return loss

    def extended():
        loss, lse = kd.forward_ex(H, W, idx, t, T, chunk, workspace=ws, **ext)
        kd.backward_ex(H, W, idx, t, lse, None, T, chunk, dW=dW, workspace=ws, **ext)
        return loss

    out = {}
    for name, fn in (("plain", plain), ("extended", extended)):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(args.steps, 1)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            loss = fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        out[name] = {"ms_median": round(times[len(times) // 2], 3), "loss": float(loss.item()),
                     "tokens_per_s": round(N / (times[len(times) // 2] * 1e-3), 1)}
        log(f"{name}: {out[name]}")
    line = {"mode": "loss_extensions", "config": {**_config_doc(cfg, args.seed),
                                                  "mask_frac": 0.1, "no_label_frac": 0.05,
                                                  "kd_weight": 0.5, "ce_weight": 0.5, "scale_T2": True},
            **out, "time_ratio_extended_over_plain":
                round(out["extended"]["ms_median"] / out["plain"]["ms_median"], 4)}
    print(json.dumps(line), flush=True)


def dense_teacher(args):
    """Dense-teacher (online) mode on --config: the student's fused forward +
    backward against full-vocabulary teacher logits (fp32 or bf16, drawn on the
    device from a seeded generator).  Reports tokens/s and the extra HBM
    stream of teacher logits (read once per pass)."""
    import numpy as np
    import torch
    import lm_head_top_amd as kd
    from synth import get_config, make_inputs
    kd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    inp = make_inputs(cfg, args.seed)
    H = torch.from_numpy(inp["H"].view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed + 1)
    tt = torch.randn((cfg.N, cfg.V), generator=g, device=dev) * 3 ** 0.5
    if args.topk_dtype == "bf16":
        tt = tt.to(torch.bfloat16)
    ws = torch.empty(kd.dense_workspace_size(cfg.N, cfg.D, cfg.V, cfg.chunk), dtype=torch.uint8,
                     device=dev)
    dW = torch.zeros((cfg.V, cfg.D), dtype=torch.float32, device=dev)

    def step():
        loss, lse, lse_t = kd.dense_forward(H, W, tt, cfg.T, cfg.chunk, workspace=ws)
        kd.dense_backward(H, W, tt, lse, lse_t, None, cfg.T, cfg.chunk, dW=dW, workspace=ws)
        return loss

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        loss = step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = 8.0 * cfg.N * cfg.D * cfg.V / (ms * 1e-3) / 1e12
    line = {"mode": "dense_teacher", "metric": "fused dense-teacher KL fwd+bwd tokens/s", "unit": "tokens/s",
            "value": round(cfg.N / (ms * 1e-3), 1), "ms_per_step": round(ms, 4), "steps": args.steps,
            "tflops": round(tflops, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "teacher_dtype": args.topk_dtype,
            "teacher_bytes_per_step": 2 * cfg.N * cfg.V * tt.element_size(),
            "peak_hbm_gib": round(torch.cuda.max_memory_allocated() / 2**30, 3),
            "loss": float(loss.item()), "config": _config_doc(cfg, args.seed)}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, choices=sorted(WORKLOAD_NAMES),
                    help="workload (default: very_long for the bench line, toy for the other modes)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="positions of the CPU-oracle sample (one 4096-position chunk of the "
                         "default workload: about 13 s of fp64 work per run on 16 host threads; "
                         "0 skips it)")
    ap.add_argument("--cpu-repeats", type=int, default=3, help="runs of the CPU-oracle sample (median)")
    ap.add_argument("--profile-steps", type=int, default=2,
                    help="steps of the separate pass, after the timed steps, whose launches are "
                         "bracketed by HIP events for the per-kernel averages")
    ap.add_argument("--inputs-cache", default=None,
                    help="directory for a .npz copy of the seeded inputs: loaded when present, "
                         "written after drawing otherwise (saves the host draw in repeated runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain fp32 copy of this many MiB before warmup, as the known "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-calibration-mib run into "
                         "profiles/traffic_<workload>.json")
    ap.add_argument("--traffic-command", default="",
                    help="with --traffic-from / --stats-from: the profiling command, recorded")
    ap.add_argument("--stats-from", nargs=2, metavar=("STATS_DIR", "OUT_MD"),
                    help="no GPU run: summarise a rocprofv3 --kernel-trace --stats folder into "
                         "OUT_MD (with the bench line from --bench-log if given)")
    ap.add_argument("--bench-log", default=None)
    ap.add_argument("--memory-sweep", action="store_true",
                    help="peak memory and time of one forward + backward for N in --sweep-n "
                         "(D=4096, V=131072, K=100, chunk=2048); prints the linear fit")
    ap.add_argument("--sweep-n", type=int, nargs="+",
                    default=[8192, 16384, 32768, 65536, 131072, 262144])
    ap.add_argument("--dense-reference", action="store_true",
                    help="plain PyTorch dense loss beside the fused one on --config "
                         "(peak memory, time)")
    ap.add_argument("--topk-writer", action="store_true",
                    help="time the teacher top-K cache writer on N x V teacher logits of --config")
    ap.add_argument("--topk-dtype", default="f32", choices=("f32", "bf16"))
    ap.add_argument("--keep-compare", action="store_true",
                    help="the fused loss beside the kept-gradient and kept-logits comparators on --config")
    ap.add_argument("--keep-modes", nargs="+", default=["fused", "kept_gradient", "kept_logits"],
                    choices=["fused", "kept_gradient", "kept_logits"])
    ap.add_argument("--dense-n", type=int, default=0,
                    help="with --dense-reference: positions to use instead of the workload's N")
    ap.add_argument("--dense-teacher", action="store_true",
                    help="the dense-teacher (full-vocabulary) mode on --config "
                         "(teacher dtype from --topk-dtype)")
    ap.add_argument("--loss-ext", action="store_true",
                    help="the loss extensions (mask, hard-label mix, T^2) beside the plain loss "
                         "on --config")
    ap.add_argument("--blas-compare", action="store_true",
                    help="the four GEMM kernels beside hipBLASLt (torch.mm) on the same shapes of --config")
    args = ap.parse_args()
    modes = (args.loss_ext, args.blas_compare, args.keep_compare, args.dense_teacher, args.memory_sweep,
             args.dense_reference, args.topk_writer)
    if args.config is None:
        args.config = "toy" if any(modes) else "very_long"
    if args.gpus != 1 and not (args.stats_from or args.traffic_from):
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the loss runs on one "
              "device, and how it would shard over several is described, not implemented",
              file=sys.stderr)
        sys.exit(2)
    if args.loss_ext:
        loss_ext(args)
        return
    if args.blas_compare:
        blas_compare(args)
        return
    if args.keep_compare or args.dense_teacher:
        (keep_compare if args.keep_compare else dense_teacher)(args)
        return
    if args.memory_sweep or args.dense_reference or args.topk_writer:
        if args.memory_sweep:
            memory_sweep(args)
        elif args.dense_reference:
            dense_reference(args)
        else:
            topk_writer(args)
        return
    if args.stats_from:
        line = None
        if args.bench_log:
            with open(args.bench_log) as f:
                cands = [ln for ln in f if ln.startswith("{") and '"metric"' in ln]
            line = cands[-1] if cands else None
        write_stats(args.stats_from[0], args.stats_from[1], args.traffic_command, line)
        return
    if args.traffic_from:
        if args.copy_calibration_mib <= 0:
            raise SystemExit("--traffic-from needs the --copy-calibration-mib the runs used")
        from synth import get_config
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.copy_calibration_mib,
                      args.traffic_command, _config_doc(get_config(args.config), args.seed))
        return

    import numpy as np
    import torch

    import lm_head_top_amd as kd
    from synth import get_config

    kd.load_library()
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    inp = load_inputs(cfg, args.seed, args.inputs_cache)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    H = torch.from_numpy(inp["H"].view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(inp["idx"]).to(dev)
    t = torch.from_numpy(inp["t"]).to(dev)
    ws = torch.empty(kd.workspace_size(cfg.N, cfg.D, cfg.V, cfg.K, cfg.chunk), dtype=torch.uint8,
                     device=dev)
    dW = torch.zeros((cfg.V, cfg.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    def step():
        loss, lse = kd.forward(H, W, idx, t, cfg.T, cfg.chunk, workspace=ws)
        dH, _ = kd.backward(H, W, idx, t, lse, None, cfg.T, cfg.chunk, dW=dW, workspace=ws)
        return loss, dH

    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib * 2**18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.reset_peak_memory_stats()
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    kd.profile_enable(None)  # the timed steps carry no per-kernel events
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # per step: start, forward done, backward done (three events on the stream per step)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        evs[i][0].record(stream)
        loss, lse = kd.forward(H, W, idx, t, cfg.T, cfg.chunk, workspace=ws)
        evs[i][1].record(stream)
        dH, _ = kd.backward(H, W, idx, t, lse, None, cfg.T, cfg.chunk, dW=dW, workspace=ws)
        evs[i][2].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    fwd_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    bwd_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
    med = lambda v: v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    peak_gib = torch.cuda.max_memory_allocated() / 2**30
    reserved_gib = torch.cuda.max_memory_reserved() / 2**30
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "hbm_gib": round(props.total_memory / 2**30, 1),
              "peak_basis": "published dense bf16: 256 CUs x 2.4 GHz x 4096 flop/clk/CU"}
    flops_step = 8.0 * cfg.N * cfg.D * cfg.V
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = cfg.N / (ms_per_step * 1e-3)
    log(f"loss {loss.item():.6f}; {ms_per_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); "
        f"{tflops:.1f} TFLOP/s = {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak; "
        f"peak {peak_gib:.2f} GiB")

    # Per-kernel averages: a separate pass whose GEMM launches are bracketed by
    # HIP events the library records on the launch stream.
    psteps = max(args.profile_steps, 1)
    kd.profile_enable(GEMM_KERNELS)
    for k in GEMM_KERNELS:
        kd.profile_read(k)  # drop anything recorded before
    for _ in range(psteps):
        step()
    torch.cuda.synchronize()
    kd.profile_enable(None)
    per_kernel = {}
    for k in GEMM_KERNELS:
        ms, n = kd.profile_read(k)
        per_kernel[k] = {"total_ms": ms, "launches": n, "avg_ms": ms / max(n, 1)}
        log(f"  {k:11s} {ms / psteps:8.3f} ms/step over {n} launches in {psteps} steps, "
            f"avg {ms / max(n, 1):.3f} ms")

    dom = max(GEMM_KERNELS, key=lambda k: per_kernel[k]["total_ms"])
    dk = per_kernel[dom]
    # each GEMM kind does 2 N D V flops per step in total, spread over its launches
    per_launch = 2.0 * cfg.N * cfg.D * cfg.V * psteps / max(dk["launches"], 1)
    achieved = per_launch / (dk["avg_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, _config_doc(cfg, args.seed)),
                "avg_launch_ms": round(dk["avg_ms"], 4),
                "flops_per_launch": per_launch}

    base = None
    if args.cpu_rows > 0:
        loss_v = float(loss.item())
        del H, W, idx, t, ws, dW, dH, lse, loss
        torch.cuda.empty_cache()
        base = cpu_baseline(inp, cfg, args.cpu_rows, args.cpu_repeats)
        log(f"cpu oracle: {base['value']:.2f} tokens/s on {base['cores']} threads ({base['cpu_model']}; "
            f"{base['blas']}); {base['sample']}")

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; H~N(0,1), W~N(0,1/D) in bf16; Zipf(1.1) teacher ids, "
                "sorted N(0,3) teacher logits)",
        "config": _config_doc(cfg, args.seed),
        "tflops": round(tflops, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "peak_hbm_gib": round(peak_gib, 3), "peak_reserved_gib": round(reserved_gib, 3),
        "device": device,
        "median_ms": {"step": round(med(step_ms), 4), "forward": round(med(fwd_ms), 4),
                      "backward": round(med(bwd_ms), 4)},
        "kernel_ms_per_step": {k: round(v["total_ms"] / psteps, 4) for k, v in per_kernel.items()},
        "roofline": roofline, "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


def load_inputs(cfg, seed, cache_dir=None):
    """The workload's seeded inputs (synth.make_inputs), optionally through an
    .npz copy in cache_dir keyed by workload and seed."""
    import numpy as np
    from synth import make_inputs
    path = None
    if cache_dir:
        path = os.path.join(cache_dir, f"kd_inputs_{cfg.name}_seed{seed}.npz")
        if os.path.exists(path):
            with np.load(path) as z:
                return {"H": z["H"], "W": z["W"], "idx": z["idx"], "t": z["t"], "cfg": cfg, "seed": seed}
    inp = make_inputs(cfg, seed)
    if path is not None:
        os.makedirs(cache_dir, exist_ok=True)
        tmp = path + f".{os.getpid()}.tmp.npz"
        np.savez(tmp, H=inp["H"], W=inp["W"], idx=inp["idx"], t=inp["t"])
        os.replace(tmp, path)
    return inp


if __name__ == "__main__":
    main()
