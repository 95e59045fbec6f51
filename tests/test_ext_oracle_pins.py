"""Pins of the loss-extension oracle (weights / mask, hard-label CE mix, T^2)
against facts that do not come from it.  Planted mistakes in its helpers
must each fail a pin."""
import numpy as np
import pytest

from oracle import kl_ext_oracle as E
from oracle import kl_oracle as O

torch = pytest.importorskip("torch")


def _case(seed, N=24, D=16, V=40, K=6):
    r = np.random.default_rng(seed)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) / np.sqrt(D)
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    t = np.sort(r.standard_normal((N, K)) * 1.7, axis=1)[:, ::-1].copy()
    y = r.integers(0, V, N).astype(np.int32)
    w = r.random(N) + 0.1
    return H, W, idx, t, y, w


def _torch_reference(H, W, idx, t, T, y, w, alpha, beta, s):
    """The definition through torch's log_softmax / gather / cross_entropy and
    its autograd, in float64."""
    Ht = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    z = Ht @ Wt.T / T
    logq = torch.log_softmax(z, dim=1)
    logp = torch.log_softmax(torch.tensor(t, dtype=torch.float64) / T, dim=1)
    kl = (logp.exp() * (logp - logq.gather(1, torch.tensor(idx, dtype=torch.int64)))).sum(dim=1)
    yt = torch.tensor(y, dtype=torch.int64)
    ce = torch.nn.functional.cross_entropy(z, yt.clamp(min=0), reduction="none") * (yt >= 0)
    wt = torch.tensor(w, dtype=torch.float64)
    loss = (wt * s * (alpha * kl + beta * ce)).sum() / wt.sum()
    loss.backward()
    return loss.item(), Ht.grad.numpy(), Wt.grad.numpy()


def pin_defaults_reduce_to_base():
    H, W, idx, t, _, _ = _case(1)
    a = E.forward_backward_ext(H, W, idx, t, 1.5)
    b = O.forward(H, W, idx, t, 1.5)
    g = O.backward(H, W, idx, t, 1.5)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(b["loss"])
    assert np.allclose(a["dH"], g["dH"], rtol=1e-10, atol=1e-14)
    assert np.allclose(a["dW"], g["dW"], rtol=1e-10, atol=1e-14)


def pin_pure_ce_is_torch_cross_entropy():
    H, W, idx, t, y, _ = _case(2)
    out = E.forward_backward_ext(H, W, idx, t, 1.0, labels=y, alpha=0.0, beta=1.0)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(Ht @ Wt.T, torch.tensor(y, dtype=torch.int64))
    ce.backward()
    assert abs(out["loss"] - ce.item()) <= 1e-10
    assert np.allclose(out["dH"], Ht.grad.numpy(), rtol=1e-8, atol=1e-12)
    assert np.allclose(out["dW"], Wt.grad.numpy(), rtol=1e-8, atol=1e-12)


def pin_mixed_weighted_loss_against_autograd(scale_T2=False):
    H, W, idx, t, y, w = _case(3)
    y[::5] = -1                      # some rows without a label
    T, alpha, beta = 1.7, 0.6, 0.4
    out = E.forward_backward_ext(H, W, idx, t, T, labels=y, weights=w, alpha=alpha, beta=beta,
                                 scale_T2=scale_T2, grad_loss=0.8)
    s = T * T if scale_T2 else 1.0
    loss, dH, dW = _torch_reference(H, W, idx, t, T, y, w, alpha, beta, s)
    assert abs(out["loss"] - loss) <= 1e-10 * abs(loss)
    assert np.allclose(out["dH"], 0.8 * dH, rtol=1e-8, atol=1e-12)
    assert np.allclose(out["dW"], 0.8 * dW, rtol=1e-8, atol=1e-12)


def pin_t2_scaling():
    H, W, idx, t, y, w = _case(4)
    a = E.forward_backward_ext(H, W, idx, t, 2.0, labels=y, weights=w, beta=0.3)
    b = E.forward_backward_ext(H, W, idx, t, 2.0, labels=y, weights=w, beta=0.3, scale_T2=True)
    assert abs(b["loss"] - 4.0 * a["loss"]) <= 1e-12 * abs(b["loss"])
    assert np.allclose(b["dH"], 4.0 * a["dH"], rtol=1e-12, atol=0)


def pin_mask_equals_subset():
    H, W, idx, t, y, _ = _case(5)
    w = np.ones(len(H))
    w[3:9] = 0.0
    keep = w > 0
    a = E.forward_backward_ext(H, W, idx, t, 1.0, labels=y, weights=w, beta=0.5)
    b = E.forward_backward_ext(H[keep], W, idx[keep], t[keep], 1.0, labels=y[keep], beta=0.5)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(b["loss"])
    assert np.all(a["dH"][~keep] == 0)
    assert np.allclose(a["dH"][keep], b["dH"], rtol=1e-10, atol=1e-14)
    assert np.allclose(a["dW"], b["dW"], rtol=1e-10, atol=1e-14)


def pin_gradient_rows_sum_to_zero():
    """Every row of G sums to zero (softmax minus probability masses)."""
    H, _, _, t, y, w = _case(6)
    # recover G from dH = G W with a square invertible W (V = D = 16)
    r = np.random.default_rng(7)
    Wsq = r.standard_normal((16, 16))
    idx = np.stack([r.choice(16, 6, replace=False) for _ in range(len(H))]).astype(np.int32)
    labels = (y % 16).astype(np.int32)
    labels[::3] = -1
    out = E.forward_backward_ext(H, Wsq, idx, t, 1.3, labels=labels, weights=w, alpha=0.7, beta=0.9)
    G = out["dH"] @ np.linalg.inv(Wsq)
    assert np.allclose(G.sum(axis=1), 0.0, atol=1e-12)


def pin_rows_form_equals_dense():
    """The per-row form (used at full size) gives the dense form's lse, row
    loss and dH rows, with the weight normaliser taken over all positions."""
    H, W, idx, t, _, _ = _case(11, N=30, V=50, K=7)
    r = np.random.default_rng(12)
    labels = r.integers(0, 50, 30).astype(np.int32)
    labels[::4] = -1
    w = r.random(30) * 2.0
    kw = dict(labels=labels, weights=w, alpha=0.6, beta=0.8, scale_T2=True, grad_loss=0.4)
    dense = E.forward_backward_ext(H, W, idx, t, 1.7, **kw)
    rows = [0, 3, 17, 29]
    part = E.rows_ext(H, W, idx, t, rows, 1.7, **kw)
    assert np.allclose(part["lse"], dense["lse"][rows], rtol=1e-13, atol=0)
    assert np.allclose(part["row_loss"], dense["row_loss"][rows], rtol=1e-12, atol=1e-15)
    assert np.allclose(part["dH"], dense["dH"][rows], rtol=1e-12, atol=1e-15)


PINS = [pin_defaults_reduce_to_base, pin_pure_ce_is_torch_cross_entropy,
        pin_mixed_weighted_loss_against_autograd, pin_t2_scaling, pin_mask_equals_subset,
        pin_gradient_rows_sum_to_zero, pin_rows_form_equals_dense]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_pin_mixed_with_t2():
    pin_mixed_weighted_loss_against_autograd(scale_T2=True)


def _mut_ce_sign(z, lse, labels):
    return -E.__dict__["_ce_rows_orig"](z, lse, labels)


def _mut_label_shift(shape, labels):
    y = np.asarray(labels, dtype=np.int64)
    Y = np.zeros(shape)
    ok = np.nonzero(y >= 0)[0]
    Y[ok, (y[ok] + 1) % shape[1]] = 1.0
    return Y


def _mut_unweighted(w):
    return np.full_like(w, 1.0 / len(w))


MUTANTS = {"ce_sign": ("_ce_rows", _mut_ce_sign), "label_shift": ("_label_onehot", _mut_label_shift),
           "ignore_weights": ("_row_weights", _mut_unweighted)}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(E.__dict__, "_ce_rows_orig", E._ce_rows)
    monkeypatch.setattr(E, attr, fn)
    failed = 0
    for pin in PINS + [lambda: pin_mixed_weighted_loss_against_autograd(True)]:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
