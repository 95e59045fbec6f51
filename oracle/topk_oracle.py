"""Plain CPU oracle of the teacher top-K cache writer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library.

The cache the loss reads is written once, offline, from the teacher's
full-vocabulary logits: per position the K largest logits and their token ids
("Distilling an LLM on One GPU", section "The two changes"; "The $250GB Memory
Spike That Killed Distillation Projects Is Now Optional", section "Offline
Top-K").  The pages do not say how equal logits are ranked or in which order
the K entries are stored; this oracle reads them as:

  * entries are ordered by logit, largest first;
  * equal logits (and -0.0 against +0.0, which compare equal) go to the lower
    token id first, so the selection is unique;
  * logits are compared exactly as given (fp32, or bf16 widened exactly).

For every row n the result is the first K entries of the vocabulary sorted by
the key (-logit[n, v], v).  NaN logits are outside the contract.

Parity pins: ``tests/test_topk_oracle_pins.py`` (brute force with Python's
sort on tie-heavy rows, constant rows, K = V, signed zeros, infinities,
permutation equivariance, and planted mistakes that each must fail a pin).
"""
from __future__ import annotations

import numpy as np

from .kl_oracle import bf16_to_f64

__all__ = ["topk_select", "widen"]


def widen(logits) -> np.ndarray:
    """fp32 arrays as fp64; uint16 arrays as bf16 bit patterns widened to fp64."""
    a = np.asarray(logits)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def _row_order(row: np.ndarray) -> np.ndarray:
    """Token ids of one row sorted by (logit descending, id ascending)."""
    ids = np.arange(row.shape[0])
    # np.lexsort sorts by the last key first: primary -row (ascending, i.e.
    # logits descending), secondary the id (ascending)
    return np.lexsort((ids, -row))


def topk_select(logits, K: int):
    """The K best (id, logit) pairs of every row, best first.

    logits: [N, V] fp32 (or uint16 bf16 bit patterns).  Returns int32 ids
    [N, K] and fp64 logits [N, K] (exact values of the inputs).
    """
    L = widen(logits)
    N, V = L.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    ids = np.empty((N, K), dtype=np.int32)
    vals = np.empty((N, K), dtype=np.float64)
    for n in range(N):
        order = _row_order(L[n])[:K]
        ids[n] = order
        vals[n] = L[n, order]
    return ids, vals
