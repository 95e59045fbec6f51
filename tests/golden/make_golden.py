"""Writes the oracle's full-problem results for the large workloads.

Runs only the fp64 oracle (oracle/) on the seeded inputs (synth/): the whole
problem, row-blocked with block = chunk, and stores
  loss, lse[N], row_kl[N]  (float32; the GPU bar is relative 1e-3)
  dW rows at a few sampled vocabulary ids (float32), dW column sums (float64)
in tests/golden/<config>_seed<seed>.npz.  Nothing here comes from the GPU path.

Usage: python tests/golden/make_golden.py toy long large_vocab [--seed 0]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import kl_oracle as O  # noqa: E402
from synth import get_config, make_inputs  # noqa: E402


def sampled_vocab_rows(V: int):
    """Vocabulary rows whose dW is stored: the Zipf head, tile edges, the tail."""
    rows = [0, 1, 2, 3, 255, 256, 257, V // 2, V - 257, V - 256, V - 2, V - 1]
    return sorted({r for r in rows if 0 <= r < V})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("configs", nargs="+")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    for name in args.configs:
        cfg = get_config(name)
        t0 = time.time()
        inp = make_inputs(cfg, args.seed)
        out = O.forward_backward_blocked(inp["H"], inp["W"], inp["idx"], inp["t"], cfg.T,
                                         block=cfg.chunk, want_grads=True)
        rows = sampled_vocab_rows(cfg.V)
        path = os.path.join(HERE, f"{name}_seed{args.seed}.npz")
        meta = {"config": name, "seed": args.seed, "N": cfg.N, "D": cfg.D, "V": cfg.V, "K": cfg.K,
                "chunk": cfg.chunk, "T": cfg.T, "grad_loss": 1.0,
                "written_by": "tests/golden/make_golden.py (fp64 oracle, row-blocked)"}
        np.savez_compressed(
            path, loss=np.float64(out["loss"]), lse=out["lse"].astype(np.float32),
            row_kl=out["row_kl"].astype(np.float32), dw_rows=np.array(rows, dtype=np.int64),
            dw=out["dW"][rows].astype(np.float32), dw_colsum=out["dW"].sum(axis=0),
            meta=np.array(json.dumps(meta)))
        print(f"{name}: loss {out['loss']:.9f} written to {path} in {time.time() - t0:.0f} s",
              flush=True)
        del out, inp


if __name__ == "__main__":
    main()
