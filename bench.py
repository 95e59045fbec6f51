#!/usr/bin/env python3
"""Benchmark: fused chunked top-K KL loss, forward + backward, on one MI355X.

One step = kd_topk_kl_forward + kd_topk_kl_backward over the whole batch of
N positions (every chunk), with inputs already resident in device memory.
Default workload: the toy LM head (N = 8192 positions, D = 4096,
V = 131072, K = 100, chunk = 1024, T = 1), synthetic seeded inputs.

Prints one JSON line on stdout; everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused top-K KL fwd+bwd tokens/s and % bf16 MFMA peak; peak HBM GiB"
# MI355X published dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
GEMM_KERNELS = ("logits_fwd", "logits_bwd", "dh", "dw")
WORKLOAD_NAMES = {"tiny": "tiny", "toy": "toy_lm_head", "large_vocab": "large_vocab_head",
                  "long": "long_context", "very_long": "very_long_context"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(inp, cfg, rows):
    """The fp64 oracle, as it stands, on the first `rows` positions of the workload."""
    import numpy as np
    from oracle import kl_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    rows = min(rows, cfg.N)
    H = inp["H"][:rows]
    idx = inp["idx"][:rows]
    t = inp["t"][:rows]
    t0 = time.perf_counter()
    out = O.forward_backward_blocked(H, inp["W"], idx, t, cfg.T, block=min(cfg.chunk, rows))
    dt = time.perf_counter() - t0
    assert np.isfinite(out["loss"])
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {cfg.N} positions of the same workload (fp64 numpy, "
                      f"row-blocked, block={min(cfg.chunk, rows)}); {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="toy", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="positions of the CPU-oracle sample (0 skips it)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the method's "
              "multi-GPU sharding is a design note, not part of this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lm_head_top_amd as kd
    from synth import get_config, make_inputs

    kd.load_library()
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, args.seed)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kd.profile_enable(GEMM_KERNELS)
    for k in GEMM_KERNELS:
        kd.profile_read(k)  # drop anything recorded before the timed region
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        loss, dH = step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kd.profile_enable(None)
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    peak_gib = torch.cuda.max_memory_allocated() / 2**30
    per_kernel = {}
    for k in GEMM_KERNELS:
        ms, n = kd.profile_read(k)
        per_kernel[k] = {"total_ms": ms, "launches": n, "avg_ms": ms / max(n, 1)}
    flops_step = 8.0 * cfg.N * cfg.D * cfg.V
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = cfg.N / (ms_per_step * 1e-3)
    log(f"loss {loss.item():.6f}; {ms_per_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); "
        f"{tflops:.1f} TFLOP/s = {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak; "
        f"peak {peak_gib:.2f} GiB")
    for k, v in per_kernel.items():
        log(f"  {k:11s} {v['total_ms'] / args.steps:8.3f} ms/step over {v['launches']} launches, "
            f"avg {v['avg_ms']:.3f} ms")

    dom = max(GEMM_KERNELS, key=lambda k: per_kernel[k]["total_ms"])
    dk = per_kernel[dom]
    # each GEMM kind does 2 N D V flops per step in total, spread over its launches
    flops_dom = 2.0 * cfg.N * cfg.D * cfg.V * args.steps
    per_launch = flops_dom / max(dk["launches"], 1)
    achieved = per_launch / (dk["avg_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "avg_launch_ms": round(dk["avg_ms"], 4),
                "flops_per_launch": per_launch}

    base = None
    if args.cpu_rows > 0:
        del H, W, idx, t, ws, dW
        torch.cuda.empty_cache()
        base = cpu_baseline(inp, cfg, args.cpu_rows)
        log(f"cpu oracle: {base['value']:.2f} tokens/s on {base['cores']} threads")

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; H~N(0,1), W~N(0,1/D) in bf16; Zipf(1.1) teacher ids, "
                "sorted N(0,3) teacher logits)",
        "config": {"workload": WORKLOAD_NAMES[cfg.name], "N": cfg.N, "D": cfg.D, "V": cfg.V,
                   "K": cfg.K, "chunk": cfg.chunk, "T": cfg.T, "seed": args.seed},
        "tflops": round(tflops, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "peak_hbm_gib": round(peak_gib, 3),
        "kernel_ms_per_step": {k: round(v["total_ms"] / args.steps, 4) for k, v in per_kernel.items()},
        "roofline": roofline, "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
