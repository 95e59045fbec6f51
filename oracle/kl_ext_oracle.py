"""Plain fp64 CPU oracle of the loss extensions: a per-position weight (a mask),
a hard-label cross-entropy term mixed with the KL term, and optional T^2
scaling.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests use it.  It shares no code with the HIP
library.

The pages report ablations over loss terms and note that packing sequences
with an all-ones attention mask costs accuracy ("The $250GB Memory Spike That
Killed Distillation Projects Is Now Optional", section "What a Single H200 GPU
Can Now Do That Once Required Four Nodes"); they do not define these
extensions, so this oracle reads them as follows.  With z = H W^T / T, lse,
the teacher distribution p over the K cached entries and KL_n exactly as in
kl_oracle:

  CE_n  = lse_n - z[n, y_n]      for a label y_n >= 0, and 0 for y_n < 0
          (cross-entropy against a hard label, on the same temperature-scaled
          logits as the KL term)
  l_n   = s (alpha KL_n + beta CE_n),   s = T^2 if scale_T2 else 1
  loss  = sum_n w_n l_n / sum_n w_n     (w_n = 1 without weights; 0 if the
                                         weights sum to 0)
  G[n, v] = g s (w_n / sum_m w_m) / T *
            ((alpha + beta [y_n >= 0]) softmax(z_n)_v
             - alpha sum_{k: idx[n,k] = v} p[n, k] - beta [v = y_n])
  dH = G W,   dW = dW_in + G^T H

With no weights, no labels, alpha = 1, beta = 0 and no T^2 scaling this is
the base loss of kl_oracle.

Parity pins: ``tests/test_ext_oracle_pins.py`` (reduction to the base oracle,
cross-entropy against torch.nn.functional.cross_entropy, the mixed and
weighted loss and its gradients against torch autograd, masked rows, the T^2
factor, the per-row form against the dense one, and planted mistakes).
"""
from __future__ import annotations

import numpy as np

from . import kl_oracle as K

__all__ = ["forward_backward_ext", "rows_ext"]


def _ce_rows(z: np.ndarray, lse: np.ndarray, labels) -> np.ndarray:
    """CE_n = lse_n - z[n, y_n] for y_n >= 0, else 0."""
    y = np.asarray(labels, dtype=np.int64)
    ok = y >= 0
    zy = np.take_along_axis(z, np.where(ok, y, 0)[:, None], axis=1)[:, 0]
    return np.where(ok, lse - zy, 0.0)


def _label_onehot(shape, labels) -> np.ndarray:
    y = np.asarray(labels, dtype=np.int64)
    Y = np.zeros(shape)
    ok = np.nonzero(y >= 0)[0]
    Y[ok, y[ok]] = 1.0
    return Y


def _row_weights(w: np.ndarray) -> np.ndarray:
    """w_n / sum_m w_m (all zero when the weights sum to zero)."""
    wsum = w.sum()
    return w / wsum if wsum != 0 else np.zeros_like(w)


def _grad_rows(z, lse, idx, p, y, r, alpha, beta, s, T, grad_loss):
    """G for the given rows: g s r_n / T ((alpha + beta [y_n >= 0]) softmax(z_n)
    - alpha sum_{k: idx[n,k]=v} p[n,k] - beta [v = y_n])."""
    n = z.shape[0]
    q = np.exp(z - lse[:, None])
    P = np.zeros_like(q)
    rows = np.repeat(np.arange(n), p.shape[1])
    np.add.at(P, (rows, np.asarray(idx, dtype=np.int64).reshape(-1)), p.reshape(-1))
    coef = alpha + beta * (y >= 0)
    Gt = coef[:, None] * q - alpha * P - beta * _label_onehot(q.shape, y)
    scale = (float(grad_loss) * s / float(T)) * r
    return scale[:, None] * Gt


def forward_backward_ext(H, W, idx, t, T: float = 1.0, labels=None, weights=None,
                         alpha: float = 1.0, beta: float = 0.0, scale_T2: bool = False,
                         grad_loss: float = 1.0, want_grads: bool = True, dW_in=None):
    """Dense form (materialises z; small problems only).  Returns dict(loss,
    lse, row_loss, and dH, dW when want_grads)."""
    Hf = K._as_f64(H)
    Wf = K._as_f64(W)
    N = Hf.shape[0]
    z = K.student_logits(Hf, Wf, T)
    kl, lse, p = K.kl_rows_from_logits(z, idx, t, T)
    y = np.full(N, -1, dtype=np.int64) if labels is None else np.asarray(labels, dtype=np.int64)
    w = np.ones(N) if weights is None else np.asarray(weights, dtype=np.float64)
    s = float(T) ** 2 if scale_T2 else 1.0
    row_loss = s * (alpha * kl + beta * _ce_rows(z, lse, y))
    r = _row_weights(w)
    loss = float((r * row_loss).sum())
    out = {"loss": loss, "lse": lse, "row_loss": row_loss}
    if want_grads:
        G = _grad_rows(z, lse, idx, p, y, r, alpha, beta, s, T, grad_loss)
        out["dH"] = G @ Wf
        out["dW"] = (0.0 if dW_in is None else np.asarray(dW_in, dtype=np.float64)) + G.T @ Hf
    return out


def rows_ext(H, W, idx, t, rows, T: float = 1.0, labels=None, weights=None,
             alpha: float = 1.0, beta: float = 0.0, scale_T2: bool = False,
             grad_loss: float = 1.0):
    """Per-row results for a sample of rows of a (possibly huge) problem: lse,
    row_loss and the dH row (each needs only that row's logits; the weight
    normaliser sum_m w_m runs over the full ``weights`` vector).  Returns
    dict(lse, row_loss, dH) in the order of ``rows``."""
    rows = np.asarray(rows, dtype=np.int64)
    N = np.asarray(H).shape[0]
    Wf = K._as_f64(W)
    Hb = K._as_f64(np.asarray(H)[rows])
    z = K.student_logits(Hb, Wf, T)
    idx_b = np.asarray(idx)[rows]
    kl, lse, p = K.kl_rows_from_logits(z, idx_b, np.asarray(t)[rows], T)
    y_all = np.full(N, -1, dtype=np.int64) if labels is None else np.asarray(labels, dtype=np.int64)
    w_all = np.ones(N) if weights is None else np.asarray(weights, dtype=np.float64)
    y = y_all[rows]
    s = float(T) ** 2 if scale_T2 else 1.0
    row_loss = s * (alpha * kl + beta * _ce_rows(z, lse, y))
    r = _row_weights(w_all)[rows]
    G = _grad_rows(z, lse, idx_b, p, y, r, alpha, beta, s, T, grad_loss)
    return {"lse": lse, "row_loss": row_loss, "dH": G @ Wf}
