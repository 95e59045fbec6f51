"""Seeded synthetic inputs for the fused chunked top-K KL distillation loss.

This module only draws random numbers and shapes them into the input tensors of
the loss; it contains none of the loss's arithmetic.  Both the fp64 oracle
(``oracle/``) and the GPU path's tests and benchmark take their inputs from
here, so the two sides always see bit-identical bf16 / int32 / fp32 data.

Workloads follow the pages' toy output-projection benchmark (hidden size 4096,
vocabulary 131,072; "Distilling an LLM on One GPU", section "The two changes")
and the gpt-oss vocabulary of 201,088 tokens (same page, section "Why
distillation recovery is expensive").  The teacher cache holds K token ids and
logits per position (top-100 on the pages, section "The two changes").

Recipe (all draws from numpy's PCG64, seeded by SeedSequence([seed, cfg_id]) and
spawned into four child streams in the order H, W, ids, logits):

* H ~ N(0, 1) drawn in float32, rounded to bf16 by round-to-nearest-even.
* W ~ N(0, 1/D) drawn in float32, rounded to bf16 the same way.
* Teacher ids: K distinct ids per position.  "uniform": uniform over [0, V).
  "zipf": ranks r ~ Zipf(s=1.1) truncated to [1, V] (draws above V rejected),
  the first K distinct ranks in draw order, id = r - 1.  "zipf_perm": the zipf
  ids sent through one seeded permutation of [0, V).
* Teacher logits: per position K draws of N(0, variance 3) in float32, sorted
  descending; slot k pairs the k-th drawn distinct id with the k-th largest
  logit.

bf16 tensors are returned as uint16 bit patterns (numpy has no bf16 dtype).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "KDConfig",
    "CONFIGS",
    "get_config",
    "make_inputs",
    "make_teacher_cache",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class KDConfig:
    """One workload: N positions, hidden size D, vocabulary V, K cached ids."""

    name: str
    N: int
    D: int
    V: int
    K: int
    chunk: int
    T: float = 1.0
    ids: str = "zipf"  # "uniform" | "zipf" | "zipf_perm"
    cfg_id: int = 0  # mixed into the seed so configs draw independent streams

    def replace(self, **kw) -> "KDConfig":
        return dataclasses.replace(self, **kw)


# The five workloads of the benchmark, plus their numeric ids for seeding.
CONFIGS = {
    "tiny": KDConfig("tiny", N=256, D=128, V=4096, K=16, chunk=64, ids="uniform", cfg_id=0),
    "toy": KDConfig("toy", N=8192, D=4096, V=131072, K=100, chunk=1024, cfg_id=1),
    "large_vocab": KDConfig("large_vocab", N=32768, D=2880, V=201088, K=100, chunk=2048, cfg_id=2),
    "long": KDConfig("long", N=32768, D=4096, V=131072, K=100, chunk=2048, cfg_id=3),
    "very_long": KDConfig("very_long", N=262144, D=4096, V=131072, K=100, chunk=4096, cfg_id=4),
}


def get_config(name: str, **overrides) -> KDConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest, ties to even); return uint16 bits.

    NaN is mapped to a quiet NaN; the generators never produce one.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # (u + 0x7FFF + lsb) >> 16 in 32-bit arithmetic: the sum wraps only for
    # NaN bit patterns (u >= 0xFFFF8001), which are overwritten below
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, cfg_id: int):
    ss = np.random.SeedSequence([int(seed), int(cfg_id)])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, std: float,
                 block_rows: int = 8192) -> np.ndarray:
    """rows x cols bf16 bits of N(0, std^2), drawn block by block (same stream)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def _first_k_distinct(cand: np.ndarray, K: int):
    """Per row: the first K distinct non-negative values of cand, in draw order.

    Returns (ids [R, K] int64, ok [R] bool); rows with fewer than K distinct
    valid values have ok False and garbage ids.
    """
    R, M = cand.shape
    order = np.argsort(cand, axis=1, kind="stable")
    sv = np.take_along_axis(cand, order, 1)
    first = np.ones_like(sv, dtype=bool)
    first[:, 1:] = sv[:, 1:] != sv[:, :-1]
    first &= sv >= 0
    pos = np.where(first, order, M)
    pos.sort(axis=1)
    ok = first.sum(axis=1) >= K
    ids = np.take_along_axis(cand, np.minimum(pos[:, :K], M - 1), 1)
    return ids, ok


def _draw_ids(rng: np.random.Generator, N: int, V: int, K: int, kind: str,
              block_rows: int = 4096) -> np.ndarray:
    if K > V:
        raise ValueError("K must not exceed V")
    out = np.empty((N, K), dtype=np.int32)
    if kind == "uniform" and K * 4 > V:
        # dense case: a random permutation prefix per row
        for n in range(N):
            out[n] = rng.permutation(V)[:K]
        return out
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        rows = np.arange(r0, r1)
        M = 4 * K if kind == "uniform" else max(4 * K, 400)
        todo = np.ones(len(rows), dtype=bool)
        while todo.any():
            idx_rows = np.nonzero(todo)[0]
            if kind == "uniform":
                cand = rng.integers(0, V, size=(len(idx_rows), M), dtype=np.int64)
            else:
                cand = rng.zipf(1.1, size=(len(idx_rows), M))
                cand = np.where(cand <= V, cand - 1, -1)
            ids, ok = _first_k_distinct(cand, K)
            out[rows[idx_rows[ok]]] = ids[ok]
            todo[idx_rows[ok]] = False
            M *= 2
    return out


def make_teacher_cache(cfg: KDConfig, seed: int = 0):
    """(idx int32 [N,K], logits float32 [N,K]) for cfg; see module recipe."""
    _, _, r_ids, r_t = _streams(seed, cfg.cfg_id)
    kind = cfg.ids
    base = "uniform" if kind == "uniform" else "zipf"
    idx = _draw_ids(r_ids, cfg.N, cfg.V, cfg.K, base)
    if kind == "zipf_perm":
        perm = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([int(seed), int(cfg.cfg_id), 7]))).permutation(cfg.V)
        idx = perm[idx].astype(np.int32)
    t = np.empty((cfg.N, cfg.K), dtype=np.float32)
    sd = np.float32(math.sqrt(3.0))
    for r0 in range(0, cfg.N, 65536):
        r1 = min(cfg.N, r0 + 65536)
        x = r_t.standard_normal((r1 - r0, cfg.K), dtype=np.float32) * sd
        t[r0:r1] = -np.sort(-x, axis=1)
    return idx, t


def make_inputs(cfg: KDConfig, seed: int = 0):
    """All inputs of one workload.

    Returns dict with H (uint16 bf16 bits [N,D]), W (uint16 bf16 bits [V,D]),
    idx (int32 [N,K]), t (float32 [N,K]) and the config.
    """
    r_h, r_w, _, _ = _streams(seed, cfg.cfg_id)
    H = _normal_bf16(r_h, cfg.N, cfg.D, 1.0)
    W = _normal_bf16(r_w, cfg.V, cfg.D, 1.0 / math.sqrt(cfg.D))
    idx, t = make_teacher_cache(cfg, seed)
    return {"H": H, "W": W, "idx": idx, "t": t, "cfg": cfg, "seed": seed}


def row_prefix(inputs: dict, n: int) -> dict:
    """The first n positions of a workload (same W); used for bounded samples."""
    cfg = inputs["cfg"].replace(N=n)
    return {"H": inputs["H"][:n], "W": inputs["W"], "idx": inputs["idx"][:n],
            "t": inputs["t"][:n], "cfg": cfg, "seed": inputs["seed"]}
