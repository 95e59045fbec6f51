"""Plain fp64 CPU oracle for the fused chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library.

What it computes: the plain dense definition.  The pages state that the fused
chunked loss changes memory use, not the objective ("The $250GB Memory Spike
That Killed Distillation Projects Is Now Optional", section "Caching Once,
Training Forever"), so the dense form is the reference.

For positions n in [0, N), vocabulary entries v in [0, V) and cache slots k in
[0, K), with bf16 inputs widened exactly to fp64:

  1. student logits  z[n, v] = (sum_d H[n, d] W[v, d]) / T
     (the LM-head projection of each chunk's hidden states is part of the
     loss: "Distilling an LLM on One GPU", section "The two changes"; "New
     distillation trick cuts training memory below single-GPU limit")
  2. student log-normaliser  lse[n] = log sum_v exp(z[n, v])   (full vocabulary)
  3. teacher distribution renormalised over the K cached entries at temperature T
        p[n, k] = exp(t[n, k]/T - logsumexp_k t[n, .]/T)
     (top-K cache of ids and logits: "Distilling an LLM on One GPU", section
     "The two changes"; "Breaking the Memory Barrier", section "Detailed
     Chronology and Technical Evolution")
  4. forward KL(teacher || student) on the teacher's support
        KL_n = sum_k p[n, k] (log p[n, k] - z[n, idx[n, k]] + lse[n]),
     with 0 * log 0 := 0
  5. loss = (1/N) sum_n KL_n
  6. gradient of the loss w.r.t. the temperature-scaled logits, carried back
     through the 1/T:
        G[n, v] = g / (N T) * (exp(z[n, v] - lse[n]) - sum_{k: idx[n,k] = v} p[n, k])
  7. dH = G W   (N x D)   and   dW = dW_in + G^T H   (V x D)

Where the pages leave a point open this oracle reads it as: forward KL
(teacher || student); the teacher renormalised over its K cached entries; the
temperature on both sides with no T^2 factor; the mean over all N positions;
no student-side renormalisation; duplicate ids as a scatter-add; a -inf
teacher logit as p = 0.

Parity pins: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (Gibbs inequality, KL = 0 special case, shift
invariance, the W = 0 closed form, cross-entropy at K = 1, full-vocabulary KL
via scipy/torch at K = V, blocked == dense, brute force and central finite
differences, gradient row sums, the temperature identity, and a sanity band).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64",
    "teacher_probs",
    "teacher_entropy_term",
    "student_logits",
    "log_normaliser",
    "kl_rows_from_logits",
    "grad_logits",
    "forward",
    "backward",
    "forward_backward_blocked",
    "rows_forward",
]


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)


# -- step 3: the teacher cache, renormalised over its K entries --------------

def teacher_probs(t, T: float) -> np.ndarray:
    """p[n, k] = softmax over the K cached teacher logits of t / T (fp64).

    A -inf teacher logit gets probability 0.
    """
    a = np.asarray(t, dtype=np.float64) / float(T)
    m = np.max(a, axis=1, keepdims=True)
    e = np.exp(a - m)
    return e / np.sum(e, axis=1, keepdims=True)


def teacher_entropy_term(p: np.ndarray) -> np.ndarray:
    """sum_k p log p per row, with 0 log 0 := 0 (the negative teacher entropy)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return plogp.sum(axis=1)


# -- steps 1-2: dense student logits and their log-normaliser -----------------

def student_logits(H, W, T: float) -> np.ndarray:
    """z = H W^T / T in fp64 (H: [n, D], W: [V, D]; bf16 bits or floats)."""
    return (_as_f64(H) @ _as_f64(W).T) / float(T)


def log_normaliser(z: np.ndarray) -> np.ndarray:
    """lse[n] = log sum_v exp(z[n, v]), max-shifted; -inf entries allowed."""
    m = np.max(z, axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        s = np.sum(np.exp(z - m), axis=1)
    return m[:, 0] + np.log(s)


# -- step 4: per-row KL given logits -------------------------------------------

def kl_rows_from_logits(z: np.ndarray, idx, t, T: float, zT_already: bool = True):
    """Per-row KL(teacher || student) from dense logits.

    z: [n, V] student logits.  If ``zT_already`` is False, z are raw logits and
    are divided by T here.  Entries of z may be +-inf (the logits-level form).
    Returns (row_kl [n], lse [n], p [n, K]).
    """
    z = np.asarray(z, dtype=np.float64)
    if not zT_already:
        z = z / float(T)
    idx = np.asarray(idx, dtype=np.int64)
    p = teacher_probs(t, T)
    lse = log_normaliser(z)
    zk = np.take_along_axis(z, idx, axis=1)
    student_logq = zk - lse[:, None]
    with np.errstate(invalid="ignore"):
        cross = np.where(p > 0, p * student_logq, 0.0).sum(axis=1)
    row_kl = teacher_entropy_term(p) - cross
    return row_kl, lse, p


# -- step 6: gradient w.r.t. the student logits --------------------------------

def grad_logits(z: np.ndarray, lse: np.ndarray, idx, p: np.ndarray, N_total: int,
                T: float, grad_loss: float = 1.0) -> np.ndarray:
    """G[n, v] = g/(N T) (softmax(z)[n, v] - sum_{k: idx[n,k]=v} p[n, k]).

    z are the temperature-scaled logits of the rows given; N_total is the number
    of positions the mean is taken over.
    """
    q = np.exp(z - lse[:, None])
    P = np.zeros_like(q)
    rows = np.repeat(np.arange(q.shape[0]), p.shape[1])
    np.add.at(P, (rows, np.asarray(idx, dtype=np.int64).reshape(-1)), p.reshape(-1))
    return (float(grad_loss) / (float(N_total) * float(T))) * (q - P)


# -- whole-problem forms --------------------------------------------------------

def forward(H, W, idx, t, T: float = 1.0):
    """Dense forward: dict(loss, lse [N], row_kl [N])."""
    z = student_logits(H, W, T)
    row_kl, lse, _ = kl_rows_from_logits(z, idx, t, T)
    return {"loss": float(np.mean(row_kl)), "lse": lse, "row_kl": row_kl}


def backward(H, W, idx, t, T: float = 1.0, grad_loss: float = 1.0, dW_in=None):
    """Dense backward: dict(dH [N, D], dW [V, D], G [N, V])."""
    Hf = _as_f64(H)
    Wf = _as_f64(W)
    z = student_logits(Hf, Wf, T)
    _, lse, p = kl_rows_from_logits(z, idx, t, T)
    G = grad_logits(z, lse, idx, p, Hf.shape[0], T, grad_loss)
    dW = G.T @ Hf
    if dW_in is not None:
        dW = dW + np.asarray(dW_in, dtype=np.float64)
    return {"dH": G @ Wf, "dW": dW, "G": G}


def forward_backward_blocked(H, W, idx, t, T: float = 1.0, block: int = 1024,
                             grad_loss: float = 1.0, want_grads: bool = True,
                             dW_in=None):
    """Row-blocked form of forward + backward (blocks of ``block`` positions).

    Each block's logits are built, used and dropped, so memory is O(block * V)
    rather than O(N * V); the per-row results are those of the dense form.
    Returns dict(loss, lse, row_kl, dH, dW).
    """
    Wf = _as_f64(W)
    N = np.asarray(H).shape[0]
    D = Wf.shape[1]
    V = Wf.shape[0]
    idx = np.asarray(idx)
    t = np.asarray(t)
    lse = np.empty(N)
    row_kl = np.empty(N)
    dH = np.empty((N, D)) if want_grads else None
    dW = None
    if want_grads:
        dW = np.zeros((V, D)) if dW_in is None else np.array(dW_in, dtype=np.float64)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        Hb = _as_f64(H[r0:r1])
        z = student_logits(Hb, Wf, T)
        kl_b, lse_b, p_b = kl_rows_from_logits(z, idx[r0:r1], t[r0:r1], T)
        lse[r0:r1] = lse_b
        row_kl[r0:r1] = kl_b
        if want_grads:
            G = grad_logits(z, lse_b, idx[r0:r1], p_b, N, T, grad_loss)
            dH[r0:r1] = G @ Wf
            dW += G.T @ Hb
        del z
    return {"loss": float(np.mean(row_kl)), "lse": lse, "row_kl": row_kl,
            "dH": dH, "dW": dW}


def rows_forward(H, W, idx, t, rows, N_total: int, T: float = 1.0,
                 grad_loss: float = 1.0):
    """Per-row results for a sample of rows of a (possibly huge) problem.

    For each row n in ``rows``: lse[n], row_kl[n] and dH[n, :] (dH needs only
    that row's logits).  N_total is the N of the full problem (it sets the
    1/N of the mean).  Returns dict(lse, row_kl, dH) in the order of ``rows``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Wf = _as_f64(W)
    Hb = _as_f64(np.asarray(H)[rows])
    z = student_logits(Hb, Wf, T)
    kl_b, lse_b, p_b = kl_rows_from_logits(z, np.asarray(idx)[rows], np.asarray(t)[rows], T)
    G = grad_logits(z, lse_b, np.asarray(idx)[rows], p_b, N_total, T, grad_loss)
    return {"lse": lse_b, "row_kl": kl_b, "dH": G @ Wf}
