"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function checks the oracle module ``o`` against mathematics or an
independent library routine and raises AssertionError on a mismatch.  The tests
run every pin on the real oracle, then plant plausible mistakes in the oracle
(on the CPU, by monkeypatching one of its functions) and check that at least
one pin fails for each planted mistake.

The pages print no worked numeric example, so the pins are closed forms,
invariants, special cases that reduce to library routines, brute force on
micro inputs and central finite differences.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import kl_oracle as O
from synth import f32_to_bf16_bits


# ---------------------------------------------------------------- helpers ---

def _rand_problem(seed, N, D, V, K, wscale=None, tscale=math.sqrt(3.0)):
    r = np.random.default_rng(seed)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) * (wscale if wscale is not None else 1 / math.sqrt(D))
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    t = -np.sort(-r.standard_normal((N, K)) * tscale, axis=1)
    return H, W, idx, t


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------------------- pins ---

def pin_gibbs(o):
    """P1: KL >= 0 for every row (sum_k q_idx <= 1 on the teacher support)."""
    for T in (1.0, 1.7):
        H, W, idx, t = _rand_problem(1, 40, 16, 64, 8, wscale=0.9)
        kl = o.forward(H, W, idx, t, T)["row_kl"]
        assert np.all(kl >= -1e-12), kl.min()
        assert np.all(kl > 1e-6)  # student is not the teacher here


def pin_zero_kl(o):
    """P2: student logits equal to the teacher's on the K set (+ a per-row
    constant) and -inf elsewhere give KL = 0 and G = 0."""
    r = np.random.default_rng(2)
    N, V, K = 5, 37, 6
    for T in (1.0, 2.5):
        idx = np.stack([r.choice(V, K, replace=False) for _ in range(N)])
        t = r.standard_normal((N, K)) * 2
        z = np.full((N, V), -np.inf)
        c = r.standard_normal(N)[:, None] * 3
        np.put_along_axis(z, idx, t + c, axis=1)
        kl, lse, p = o.kl_rows_from_logits(z, idx, t, T, zT_already=False)
        assert np.all(np.abs(kl) <= 1e-13), kl
        G = o.grad_logits(z / T, lse, idx, p, N, T)
        assert np.all(np.abs(G) <= 1e-15)


def pin_shift_invariance(o):
    """P3: z -> z + c_n and t -> t + c'_n leave KL and G unchanged (this also
    makes stored logits and stored log-probabilities equivalent)."""
    r = np.random.default_rng(3)
    N, V, K, T = 7, 50, 9, 1.3
    z = r.standard_normal((N, V)) * 2
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(N)])
    t = r.standard_normal((N, K)) * 2
    kl0, lse0, p0 = o.kl_rows_from_logits(z, idx, t, T, zT_already=False)
    G0 = o.grad_logits(z / T, lse0, idx, p0, N, T)
    c1 = r.standard_normal((N, 1)) * 50
    c2 = r.standard_normal((N, 1)) * 50
    kl1, lse1, p1 = o.kl_rows_from_logits(z + c1, idx, t + c2, T, zT_already=False)
    G1 = o.grad_logits((z + c1) / T, lse1, idx, p1, N, T)
    assert np.allclose(kl0, kl1, rtol=1e-10, atol=1e-12)
    assert np.allclose(G0, G1, rtol=1e-9, atol=1e-15)


def pin_zero_weight_closed_form(o):
    """P4: W = 0 gives uniform student q = 1/V, so KL_n = log V - H(p_n),
    G = (1/V - P)/(N T), dH = 0, dW = G^T H."""
    N, D, V, K, T = 6, 5, 23, 4, 1.5
    H, _, idx, t = _rand_problem(4, N, D, V, K)
    W = np.zeros((V, D))
    p = scipy.special.softmax(t / T, axis=1)
    ent = -(p * np.log(p)).sum(axis=1)
    out = o.forward(H, W, idx, t, T)
    assert np.allclose(out["row_kl"], math.log(V) - ent, rtol=1e-13, atol=1e-13)
    assert np.allclose(out["lse"], math.log(V), rtol=1e-14)
    g = o.backward(H, W, idx, t, T)
    Gref = np.full((N, V), 1.0 / V)
    for n in range(N):
        for k in range(K):
            Gref[n, idx[n, k]] -= p[n, k]
    Gref /= N * T
    assert np.allclose(g["G"], Gref, rtol=1e-12, atol=1e-16)
    assert np.all(g["dH"] == 0)
    assert np.allclose(g["dW"], Gref.T @ H, rtol=1e-12, atol=1e-16)


def pin_k1_cross_entropy(o):
    """P5: K = 1 is cross-entropy on the cached id; checked with torch's
    cross_entropy and its autograd (CPU, fp64), loss and both gradients."""
    torch = pytest.importorskip("torch")
    N, D, V = 9, 12, 40
    H, W, idx, t = _rand_problem(5, N, D, V, 1, wscale=0.7)
    out = o.forward(H, W, idx, t, 1.0)
    g = o.backward(H, W, idx, t, 1.0)
    Ht = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    tgt = torch.tensor(idx[:, 0], dtype=torch.int64)
    ce = torch.nn.functional.cross_entropy(Ht @ Wt.T, tgt, reduction="none")
    assert np.allclose(out["row_kl"], ce.detach().numpy(), rtol=1e-12, atol=1e-13)
    ce.mean().backward()
    assert _rel(g["dH"], Ht.grad.numpy()) < 1e-12
    assert _rel(g["dW"], Wt.grad.numpy()) < 1e-12


def pin_full_vocab_kl(o):
    """P6: K = V with the ids a permutation is the full-vocabulary
    KL(p || q); checked with scipy.special.rel_entr and torch kl_div."""
    torch = pytest.importorskip("torch")
    N, D, V, T = 4, 6, 11, 1.0
    r = np.random.default_rng(6)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) * 0.5
    idx = np.stack([r.permutation(V) for _ in range(N)])
    t = r.standard_normal((N, V)) * 1.5
    out = o.forward(H, W, idx, t, T)
    p = np.zeros((N, V))
    np.put_along_axis(p, idx, scipy.special.softmax(t, axis=1), axis=1)
    q = scipy.special.softmax(H @ W.T, axis=1)
    ref = scipy.special.rel_entr(p, q).sum(axis=1)
    assert np.allclose(out["row_kl"], ref, rtol=1e-11, atol=1e-13)
    kd = torch.nn.functional.kl_div(torch.tensor(np.log(q)), torch.tensor(np.log(p)),
                                    reduction="batchmean", log_target=True)
    assert abs(out["loss"] - kd.item()) < 1e-12


def pin_blocked_equals_dense(o):
    """P7: the row-blocked form equals the dense form for any block size,
    including 1, a ragged size and one block of all rows."""
    N, D, V, K, T = 23, 10, 57, 5, 1.25
    H, W, idx, t = _rand_problem(7, N, D, V, K, wscale=0.6)
    f = o.forward(H, W, idx, t, T)
    b = o.backward(H, W, idx, t, T, grad_loss=0.75)
    for blk in (1, 7, 64, N):
        r = o.forward_backward_blocked(H, W, idx, t, T, block=blk, grad_loss=0.75)
        assert abs(r["loss"] - f["loss"]) <= 1e-12 * abs(f["loss"])
        assert np.allclose(r["lse"], f["lse"], rtol=1e-13)
        assert _rel(r["dH"], b["dH"]) < 1e-12
        assert _rel(r["dW"], b["dW"]) < 1e-12
    rows = [0, 5, 22]
    s = o.rows_forward(H, W, idx, t, rows, N, T, grad_loss=0.75)
    assert np.allclose(s["row_kl"], f["row_kl"][rows], rtol=1e-13)
    assert _rel(s["dH"], b["dH"][rows]) < 1e-12


def _brute_loss(H, W, idx, t, T):
    """Pure-Python loops straight from the definition (micro sizes only)."""
    N, D = len(H), len(H[0])
    V, K = len(W), len(idx[0])
    total = 0.0
    for n in range(N):
        z = []
        for v in range(V):
            acc = 0.0
            for d in range(D):
                acc += H[n][d] * W[v][d]
            z.append(acc / T)
        mz = max(z)
        lse = mz + math.log(sum(math.exp(x - mz) for x in z))
        a = [t[n][k] / T for k in range(K)]
        ma = max(a)
        la = ma + math.log(sum(math.exp(x - ma) for x in a))
        for k in range(K):
            pk = math.exp(a[k] - la)
            total += pk * ((a[k] - la) - (z[idx[n][k]] - lse))
    return total / N


def pin_brute_force_and_finite_differences(o):
    """P8: micro inputs: the loss equals pure-Python loops; dH and dW equal
    central finite differences of the loss (step 1e-6) on 20 entries each."""
    N, D, V, K = 6, 8, 32, 5
    for T in (1.0, 2.0):
        H, W, idx, t = _rand_problem(8, N, D, V, K, wscale=0.8)
        out = o.forward(H, W, idx, t, T)
        bl = _brute_loss(H.tolist(), W.tolist(), idx.tolist(), t.tolist(), T)
        assert abs(out["loss"] - bl) <= 1e-12 * abs(bl)
        g = o.backward(H, W, idx, t, T)
        r = np.random.default_rng(80)
        h = 1e-6
        for _ in range(20):
            n, d = r.integers(N), r.integers(D)
            Hp, Hm = H.copy(), H.copy()
            Hp[n, d] += h
            Hm[n, d] -= h
            fd = (_brute_loss(Hp.tolist(), W.tolist(), idx.tolist(), t.tolist(), T)
                  - _brute_loss(Hm.tolist(), W.tolist(), idx.tolist(), t.tolist(), T)) / (2 * h)
            assert abs(fd - g["dH"][n, d]) <= 1e-6 * max(abs(fd), 1e-3), (n, d, fd, g["dH"][n, d])
            v, d = r.integers(V), r.integers(D)
            Wp, Wm = W.copy(), W.copy()
            Wp[v, d] += h
            Wm[v, d] -= h
            fd = (_brute_loss(H.tolist(), Wp.tolist(), idx.tolist(), t.tolist(), T)
                  - _brute_loss(H.tolist(), Wm.tolist(), idx.tolist(), t.tolist(), T)) / (2 * h)
            assert abs(fd - g["dW"][v, d]) <= 1e-6 * max(abs(fd), 1e-3), (v, d, fd, g["dW"][v, d])


def pin_gradient_structure(o):
    """P9: each row of G sums to 0 (softmax and p both sum to 1), so
    sum_v dW[v, :] = 0; with all W rows equal, dH = 0."""
    N, D, V, K, T = 12, 9, 45, 7, 1.1
    H, W, idx, t = _rand_problem(9, N, D, V, K, wscale=0.9)
    g = o.backward(H, W, idx, t, T)
    assert np.abs(g["G"].sum(axis=1)).max() < 1e-16 * V * 10
    assert np.abs(g["dW"].sum(axis=0)).max() < 1e-14
    Weq = np.tile(W[:1], (V, 1))
    g2 = o.backward(H, Weq, idx, t, T)
    assert np.abs(g2["dH"]).max() < 1e-14


def pin_temperature_identity(o):
    """P10: the loss at temperature T equals the loss at T = 1 with W/T and
    t/T; dH is the same and dW scales by 1/T (chain rule)."""
    N, D, V, K, T = 8, 7, 30, 6, 2.7
    H, W, idx, t = _rand_problem(10, N, D, V, K, wscale=1.5)
    a = o.forward(H, W, idx, t, T)
    b = o.forward(H, W / T, idx, t / T, 1.0)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(a["loss"])
    ga = o.backward(H, W, idx, t, T)
    gb = o.backward(H, W / T, idx, t / T, 1.0)
    assert _rel(ga["dH"], gb["dH"]) < 1e-12
    assert _rel(ga["dW"], gb["dW"] / T) < 1e-12
    # T actually matters
    c = o.forward(H, W, idx, t, 1.0)
    assert abs(c["loss"] - a["loss"]) > 1e-3


def pin_torch_autograd_general(o):
    """P12: general K, T != 1, grad_loss != 1: loss, dH and dW equal torch's
    log_softmax + gather + kl_div with autograd (CPU, fp64)."""
    torch = pytest.importorskip("torch")
    N, D, V, K, T, g = 10, 14, 60, 7, 1.6, 0.37
    H, W, idx, t = _rand_problem(12, N, D, V, K, wscale=0.8)
    out = o.forward(H, W, idx, t, T)
    gr = o.backward(H, W, idx, t, T, grad_loss=g)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    logq = torch.log_softmax((Ht @ Wt.T) / T, dim=1)
    logq_k = torch.gather(logq, 1, torch.tensor(idx, dtype=torch.int64))
    logp = torch.log_softmax(torch.tensor(t) / T, dim=1)
    loss = torch.nn.functional.kl_div(logq_k, logp, reduction="batchmean", log_target=True)
    assert abs(out["loss"] - loss.item()) <= 1e-12 * abs(loss.item())
    (g * loss).backward()
    assert _rel(gr["dH"], Ht.grad.numpy()) < 1e-12
    assert _rel(gr["dW"], Wt.grad.numpy()) < 1e-12


def pin_sanity_band(o):
    """P11 (sanity only): with z ~ N(0, 1) independent of the teacher,
    E[KL_n] ~ log V + 1/2 - H(p)."""
    N, D, V, K = 64, 256, 8192, 32
    r = np.random.default_rng(11)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) / math.sqrt(D)
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(N)])
    t = -np.sort(-r.standard_normal((N, K)) * math.sqrt(3), axis=1)
    kl = o.forward(H, W, idx, t, 1.0)["row_kl"]
    p = scipy.special.softmax(t, axis=1)
    ent = -(p * np.log(p)).sum(axis=1)
    assert abs(kl.mean() - (math.log(V) + 0.5 - ent.mean())) < 0.2


def pin_closed_form_two_word(o):
    """Hand-derived case: D = V = 2, W = I, H = [[1, 0]], K = 1, id 0.
    z = [1, 0]; q0 = sigmoid(1); KL = log(1 + e^-1); G = [q0 - 1, 1 - q0];
    dH = G; dW = [[q0 - 1, 0], [1 - q0, 0]]."""
    H = np.array([[1.0, 0.0]])
    W = np.eye(2)
    idx = np.array([[0]])
    t = np.array([[0.3]])
    out = o.forward(H, W, idx, t, 1.0)
    assert abs(out["loss"] - math.log1p(math.exp(-1.0))) < 1e-15
    s = 1.0 / (1.0 + math.exp(-1.0))
    g = o.backward(H, W, idx, t, 1.0)
    assert np.allclose(g["dH"], [[s - 1, 1 - s]], rtol=1e-14)
    assert np.allclose(g["dW"], [[s - 1, 0], [1 - s, 0]], rtol=1e-14)


def pin_duplicate_ids_scatter_add(o):
    """Duplicate ids in a row act as one entry holding the summed
    probability (scatter-add): the result equals the merged cache."""
    N, D, V, T = 3, 4, 9, 1.0
    r = np.random.default_rng(13)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D))
    idx = np.array([[2, 2, 5], [0, 8, 0], [1, 3, 4]])
    t = np.array([[1.0, 0.5, -1.0], [0.2, 0.1, 0.0], [0.0, 0.0, 0.0]])
    g = o.backward(H, W, idx, t, T)
    p = scipy.special.softmax(t, axis=1)
    z = H @ W.T
    q = scipy.special.softmax(z, axis=1)
    P = np.zeros((N, V))
    for n in range(N):
        for k in range(3):
            P[n, idx[n, k]] += p[n, k]
    G = (q - P) / N
    assert np.allclose(g["G"], G, rtol=1e-12, atol=1e-16)


PINS = [pin_gibbs, pin_zero_kl, pin_shift_invariance, pin_zero_weight_closed_form,
        pin_k1_cross_entropy, pin_full_vocab_kl, pin_blocked_equals_dense,
        pin_brute_force_and_finite_differences, pin_gradient_structure,
        pin_temperature_identity, pin_torch_autograd_general, pin_sanity_band,
        pin_closed_form_two_word, pin_duplicate_ids_scatter_add]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O)


def test_bf16_widening_is_exact():
    # includes a subnormal (0x0021 = 33 * 2^-133) and the largest finite bf16
    bits = np.array([0x3F80, 0xBC00, 0x0021, 0x7F7F, 0xBFC0], dtype=np.uint16)
    want = [1.0, -0.0078125, 33 * 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -1.5]
    assert O.bf16_to_f64(bits).tolist() == want
    x = np.array(want[:2] + want[3:], dtype=np.float32)
    assert np.array_equal(O.bf16_to_f64(f32_to_bf16_bits(x)), x.astype(np.float64))


def test_minus_inf_teacher_logit_contributes_nothing():
    """A -inf teacher logit gets p = 0 and adds nothing (0 log 0 := 0)."""
    r = np.random.default_rng(14)
    H = r.standard_normal((3, 5))
    W = r.standard_normal((12, 5))
    idx = np.array([[1, 4, 7], [0, 2, 3], [9, 10, 11]])
    t = np.array([[0.5, -np.inf, 0.1], [1.0, 2.0, -np.inf], [0.0, 1.0, 2.0]])
    a = O.forward(H, W, idx, t, 1.0)
    b = O.forward(H, W, idx[:, [0, 2]][:1], t[:1, [0, 2]], 1.0)
    assert np.isfinite(a["row_kl"]).all()
    assert abs(a["row_kl"][0] - b["row_kl"][0]) < 1e-13


# ------------------------------------------------ planted-mistake checks ---

def _mut_drop_lse(z, idx, t, T, zT_already=True):
    z = np.asarray(z, dtype=np.float64)
    if not zT_already:
        z = z / float(T)
    p = O.teacher_probs(t, T)
    lse = O.log_normaliser(z)
    zk = np.take_along_axis(z, np.asarray(idx, dtype=np.int64), axis=1)
    return O.teacher_entropy_term(p) - (p * zk).sum(1), lse, p


def _mut_gather_sign(z, idx, t, T, zT_already=True):
    z = np.asarray(z, dtype=np.float64)
    if not zT_already:
        z = z / float(T)
    p = O.teacher_probs(t, T)
    lse = O.log_normaliser(z)
    zk = np.take_along_axis(z, np.asarray(idx, dtype=np.int64), axis=1)
    return O.teacher_entropy_term(p) + (p * (zk - lse[:, None])).sum(1), lse, p


def _mut_no_entropy(z, idx, t, T, zT_already=True):
    z = np.asarray(z, dtype=np.float64)
    if not zT_already:
        z = z / float(T)
    p = O.teacher_probs(t, T)
    lse = O.log_normaliser(z)
    zk = np.take_along_axis(z, np.asarray(idx, dtype=np.int64), axis=1)
    return -(p * (zk - lse[:, None])).sum(1), lse, p


def _mut_teacher_no_T(t, T):
    return scipy.special.softmax(np.asarray(t, dtype=np.float64), axis=1)


def _mut_teacher_unnormalised(t, T):
    return np.exp(np.asarray(t, dtype=np.float64) / T)


def _make_grad_mut(kind):
    def g(z, lse, idx, p, N_total, T, grad_loss=1.0):
        q = np.exp(z - lse[:, None])
        P = np.zeros_like(q)
        ii = np.asarray(idx, dtype=np.int64)
        if kind == "shift_index":
            ii = (ii + 1) % q.shape[1]
        rows = np.repeat(np.arange(q.shape[0]), p.shape[1])
        np.add.at(P, (rows, ii.reshape(-1)), p.reshape(-1))
        scale = float(grad_loss) / (float(N_total) * float(T))
        if kind == "no_T":
            scale *= T
        if kind == "no_N":
            scale *= N_total
        if kind == "sign":
            return scale * (P - q)
        if kind == "no_grad_loss":
            scale /= grad_loss
        return scale * (q - P)
    return g


def _mut_lse_mean_over_V(z):
    m = np.max(z, axis=1, keepdims=True)
    return m[:, 0] + np.log(np.mean(np.exp(z - m), axis=1))


def _mut_logits_transposed_scale(H, W, T):
    return (O._as_f64(H) @ O._as_f64(W).T) * float(T)


MUTANTS = {
    "drop_lse": ("kl_rows_from_logits", _mut_drop_lse),
    "gather_sign": ("kl_rows_from_logits", _mut_gather_sign),
    "no_entropy": ("kl_rows_from_logits", _mut_no_entropy),
    "teacher_no_T": ("teacher_probs", _mut_teacher_no_T),
    "teacher_unnormalised": ("teacher_probs", _mut_teacher_unnormalised),
    "grad_shift_index": ("grad_logits", _make_grad_mut("shift_index")),
    "grad_no_T": ("grad_logits", _make_grad_mut("no_T")),
    "grad_no_N": ("grad_logits", _make_grad_mut("no_N")),
    "grad_sign": ("grad_logits", _make_grad_mut("sign")),
    "grad_ignores_grad_loss": ("grad_logits", _make_grad_mut("no_grad_loss")),
    "lse_mean_not_sum": ("log_normaliser", _mut_lse_mean_over_V),
    "logits_times_T": ("student_logits", _mut_logits_transposed_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = []
    for pin in PINS:
        try:
            pin(O)
        except Exception as e:  # AssertionError, or a shape/NaN error
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"planted mistake {name} passed every pin"
