"""Loss extensions on the GPU (per-position weights, a hard-label
cross-entropy term mixed with the KL term, T^2 scaling) against the oracle of
the extended loss, and agreement of the extended entry points at their
neutral settings with the plain ones."""
import numpy as np
import pytest

from oracle import kl_ext_oracle as E
from synth import get_config, make_inputs
from synth.inputs import KDConfig
from tests.kdcase import GRAD_RTOL, LOSS_RTOL, bf16_tensor_to_f64, rel, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def _run_ext(inp, T, chunk, labels=None, weights=None, alpha=1.0, beta=0.0, scale_T2=False,
             grad_loss=None, dW0=None):
    import torch
    import lm_head_top_amd as kd
    H, W, idx, t = to_device(inp)
    y = None if labels is None else torch.from_numpy(np.asarray(labels, np.int32)).cuda()
    w = None if weights is None else torch.from_numpy(np.asarray(weights, np.float32)).cuda()
    kw = dict(row_weight=w, labels=y, kd_weight=alpha, ce_weight=beta, scale_T2=scale_T2)
    loss, lse, row_loss = kd.forward_ex(H, W, idx, t, T, chunk, want_row_loss=True, **kw)
    g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    dW = None if dW0 is None else torch.from_numpy(dW0.astype(np.float32)).cuda()
    dH, dW = kd.backward_ex(H, W, idx, t, lse, g, T, chunk, dW=dW, **kw)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
            "row_loss": row_loss.double().cpu().numpy(), "dH": bf16_tensor_to_f64(dH),
            "dW": dW.double().cpu().numpy()}


def _compare(out, ref, what):
    scale = max(abs(ref["loss"]), 1e-6)
    lr = abs(out["loss"] - ref["loss"]) / scale
    rl = np.max(np.abs(out["row_loss"] - ref["row_loss"]) / np.maximum(np.abs(ref["row_loss"]), 1.0))
    le = np.max(np.abs(out["lse"] - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0))
    eh, ew = rel(out["dH"], ref["dH"]), rel(out["dW"], ref["dW"])
    say(f"  {what}: loss gpu={out['loss']:.7g} oracle={ref['loss']:.7g} rel={lr:.2e}; "
        f"row_loss {rl:.2e} lse {le:.2e}; dH {eh:.2e} dW {ew:.2e}")
    assert lr <= LOSS_RTOL and rl <= LOSS_RTOL and le <= LOSS_RTOL
    assert eh <= GRAD_RTOL and ew <= GRAD_RTOL


CASES = {
    # name: (config, T, grad_loss, alpha, beta, scale_T2, label recipe, weight recipe)
    "tiny_ce_mix": (get_config("tiny"), 1.0, None, 0.5, 0.5, False, "all", None),
    "ragged_mask_T2": (KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, T=2.0, ids="uniform",
                                cfg_id=7), 2.0, 0.37, 1.0, 0.0, True, None, "mask"),
    "ragged_labels_some_missing": (KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, T=2.0,
                                            ids="uniform", cfg_id=7), 2.0, None, 0.7, 0.3, True,
                                   "some_missing", "weights"),
    "ce_only": (KDConfig("ce", N=300, D=136, V=1000, K=16, chunk=128, T=1.0, ids="uniform", cfg_id=8),
                1.0, None, 0.0, 1.0, False, "all", None),
    # K at its limit plus a label: 257 entries per position (several load
    # rounds and the direct-scatter path of the bucketing kernel)
    "max_k_with_labels": (KDConfig("maxk", N=300, D=64, V=2000, K=256, chunk=256, T=1.0, ids="uniform",
                                   cfg_id=10), 1.5, 0.8, 0.5, 0.5, True, "some_missing", "weights"),
}


def _labels(recipe, N, V, idx, rng):
    if recipe is None:
        return None
    y = rng.integers(0, V, size=N)
    if recipe == "some_missing":
        y[rng.random(N) < 0.2] = -1
        y[::17] = idx[::17, 0]        # a label that is also a cached id
    return y


def _weights(recipe, N, rng):
    if recipe is None:
        return None
    if recipe == "mask":
        w = (rng.random(N) < 0.7).astype(np.float64)
        w[:5] = 0.0
        return w
    return rng.random(N) * 2.0


@pytest.mark.parametrize("name", sorted(CASES))
def test_ext_matches_oracle(name):
    cfg, T, g, alpha, beta, t2, lab, wr = CASES[name]
    say(f"case ext {name}: N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} T={T} "
        f"alpha={alpha} beta={beta} T2={t2} labels={lab} weights={wr}")
    inp = make_inputs(cfg, 3)
    rng = np.random.default_rng(21)
    y = _labels(lab, cfg.N, cfg.V, np.asarray(inp["idx"]), rng)
    w = _weights(wr, cfg.N, rng)
    if w is not None:
        w = w.astype(np.float32).astype(np.float64)
    dW0 = np.random.default_rng(1).standard_normal((cfg.V, cfg.D)) * 1e-3
    out = _run_ext(inp, T, cfg.chunk, labels=y, weights=w, alpha=alpha, beta=beta, scale_T2=t2,
                   grad_loss=g, dW0=dW0)
    ref = E.forward_backward_ext(inp["H"], inp["W"], inp["idx"], inp["t"], T, labels=y, weights=w,
                                 alpha=alpha, beta=beta, scale_T2=t2,
                                 grad_loss=1.0 if g is None else g,
                                 dW_in=dW0.astype(np.float32).astype(np.float64))
    _compare(out, ref, name)


def _sweep_cases(n=8, seed=20261204):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(r.integers(1, 1200))
        D = 8 * int(r.integers(1, 65))
        V = int(r.integers(40, 5001))
        K = int(r.integers(1, min(V, 256) + 1))
        chunk = int(r.integers(16, N + 65))
        T = float(r.choice([0.5, 1.0, 2.0]))
        alpha, beta = (float(x) for x in r.choice([(1.0, 0.0), (0.5, 0.5), (0.0, 1.0), (0.8, 0.3)]))
        out.append((i, N, D, V, K, chunk, T, alpha, beta, bool(r.integers(0, 2)),
                    str(r.choice(["all", "some_missing", "none"])), str(r.choice(["mask", "weights", "none"])),
                    None if i % 2 else 0.6))
    return out


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"s{c[0]}")
def test_ext_sweep(case):
    """A seeded sweep of shapes and loss settings (weights or a mask or none,
    labels all, some missing or none, the KL / CE mix, T^2) against the
    extended oracle."""
    i, N, D, V, K, chunk, T, alpha, beta, t2, lab, wr, g = case
    say(f"case ext sweep {i}: N={N} D={D} V={V} K={K} chunk={chunk} T={T} alpha={alpha} beta={beta} "
        f"T2={t2} labels={lab} weights={wr} grad={g}")
    cfg = KDConfig("sweep", N=N, D=D, V=V, K=K, chunk=chunk, T=T, ids="uniform", cfg_id=11)
    inp = make_inputs(cfg, 200 + i)
    rng = np.random.default_rng(300 + i)
    y = _labels(None if lab == "none" else lab, N, V, np.asarray(inp["idx"]), rng)
    w = _weights(None if wr == "none" else wr, N, rng)
    if w is not None:
        w = w.astype(np.float32).astype(np.float64)
        if not w.any():
            w[0] = 1.0
    out = _run_ext(inp, T, chunk, labels=y, weights=w, alpha=alpha, beta=beta, scale_T2=t2, grad_loss=g)
    ref = E.forward_backward_ext(inp["H"], inp["W"], inp["idx"], inp["t"], T, labels=y, weights=w,
                                 alpha=alpha, beta=beta, scale_T2=t2, grad_loss=1.0 if g is None else g)
    _compare(out, ref, f"sweep {i}")


def test_all_zero_weights_give_zero_loss_and_gradients():
    cfg = KDConfig("zero", N=200, D=64, V=700, K=8, chunk=128, T=1.0, ids="uniform", cfg_id=9)
    say("case ext all-zero weights")
    inp = make_inputs(cfg, 4)
    out = _run_ext(inp, 1.0, cfg.chunk, weights=np.zeros(cfg.N))
    assert out["loss"] == 0.0
    assert not out["dH"].any() and not out["dW"].any()


def test_neutral_ext_equals_plain_entry_points():
    """Without weights and labels, kd_weight 1 and no T^2 the extended entry
    points run the same kernels on the same values: bitwise-equal results."""
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("toy")
    say(f"case ext neutral vs plain, toy: N={cfg.N} D={cfg.D} V={cfg.V}")
    inp = make_inputs(cfg, 0)
    H, W, idx, t = to_device(inp)
    loss_p, lse_p = kd.forward(H, W, idx, t, cfg.T, cfg.chunk)
    dH_p, dW_p = kd.backward(H, W, idx, t, lse_p, None, cfg.T, cfg.chunk)
    loss_e, lse_e = kd.forward_ex(H, W, idx, t, cfg.T, cfg.chunk)
    dH_e, dW_e = kd.backward_ex(H, W, idx, t, lse_e, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(loss_p, loss_e) and torch.equal(lse_p, lse_e)
    assert torch.equal(dH_p, dH_e) and torch.equal(dW_p, dW_e)


def test_mask_at_full_size_matches_the_masked_subset():
    """Toy LM head with a 0/1 mask over half the positions.  A 0/1 weight
    turns the loss into the mean over the kept positions, so loss, dW and the
    kept rows of dH equal the plain entry points run on the kept positions
    alone, and the masked rows of dH are exactly zero."""
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("toy")
    say(f"case ext mask at full size: N={cfg.N} D={cfg.D} V={cfg.V}")
    inp = make_inputs(cfg, 0)
    H, W, idx, t = to_device(inp)
    rng = np.random.default_rng(5)
    keep = np.sort(rng.choice(cfg.N, size=cfg.N // 2, replace=False))
    w = np.zeros(cfg.N, np.float32)
    w[keep] = 1.0
    wt = torch.from_numpy(w).cuda()
    loss_m, lse_m = kd.forward_ex(H, W, idx, t, cfg.T, cfg.chunk, row_weight=wt)
    dH_m, dW_m = kd.backward_ex(H, W, idx, t, lse_m, None, cfg.T, cfg.chunk, row_weight=wt)
    kt = torch.from_numpy(keep).cuda()
    Hs, idxs, ts = H[kt].contiguous(), idx[kt].contiguous(), t[kt].contiguous()
    loss_s, lse_s = kd.forward(Hs, W, idxs, ts, cfg.T, cfg.chunk)
    dH_s, dW_s = kd.backward(Hs, W, idxs, ts, lse_s, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    lr = abs(loss_m.item() - loss_s.item()) / abs(loss_s.item())
    eh = rel(bf16_tensor_to_f64(dH_m[kt]), bf16_tensor_to_f64(dH_s))
    ew = float((dW_m.double() - dW_s.double()).norm() / dW_s.double().norm())
    dead = float(dH_m.float()[torch.from_numpy(w == 0).cuda()].abs().max().item())
    say(f"  loss rel {lr:.2e}; dH (kept rows) {eh:.2e}; dW {ew:.2e}; max |dH| on masked rows {dead}")
    assert lr <= LOSS_RTOL and eh <= GRAD_RTOL and ew <= GRAD_RTOL
    assert dead == 0.0


def test_ext_full_size_large_vocab_sampled_rows():
    """Large-vocabulary workload (N=32768, D=2880, V=201088, chunk 2048) with
    weights (10% zero), labels (5% missing, some in the vocabulary's tail
    tile and at V - 1), kd 0.6 / ce 0.4 and T = 2 with T^2: sampled rows
    (lse, row loss, dH row) against the oracle's per-row form, the loss
    against the weighted mean of the kernel's own row losses, and the columns
    of dW summing to zero (every row of G does)."""
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("large_vocab")
    T = 2.0
    say(f"case ext full size large_vocab: N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} T={T}")
    inp = make_inputs(cfg, 0)
    rng = np.random.default_rng(31)
    y = rng.integers(0, cfg.V, cfg.N).astype(np.int32)
    y[rng.random(cfg.N) < 0.05] = -1
    tail = rng.choice(cfg.N, 64, replace=False)
    y[tail] = rng.integers(200960, cfg.V, 64)
    y[tail[:4]] = cfg.V - 1
    w = (rng.random(cfg.N) * 2.0).astype(np.float32)
    w[rng.random(cfg.N) < 0.1] = 0.0
    rows = sorted(set([0, cfg.N - 1] + tail[:3].tolist() + np.nonzero(y < 0)[0][:2].tolist()
                      + np.nonzero(w == 0)[0][:1].tolist() + rng.integers(0, cfg.N, 3).tolist()))
    H, W, idx, t = to_device(inp)
    yt = torch.from_numpy(y).cuda()
    wt = torch.from_numpy(w).cuda()
    kw = dict(row_weight=wt, labels=yt, kd_weight=0.6, ce_weight=0.4, scale_T2=True)
    loss, lse, row_loss = kd.forward_ex(H, W, idx, t, T, cfg.chunk, want_row_loss=True, **kw)
    dH, dW = kd.backward_ex(H, W, idx, t, lse, None, T, cfg.chunk, **kw)
    torch.cuda.synchronize()
    ref = E.rows_ext(inp["H"], inp["W"], inp["idx"], inp["t"], rows, T, labels=y, weights=w.astype(np.float64),
                     alpha=0.6, beta=0.4, scale_T2=True)
    g_lse = lse.double().cpu().numpy()[rows]
    g_rl = row_loss.double().cpu().numpy()[rows]
    g_dh = bf16_tensor_to_f64(dH[rows])
    e_lse = np.max(np.abs(g_lse - ref["lse"]) / np.abs(ref["lse"]))
    e_rl = np.max(np.abs(g_rl - ref["row_loss"]) / np.maximum(np.abs(ref["row_loss"]), 1.0))
    e_dh = rel(g_dh, ref["dH"])
    say(f"  rows {rows}: lse rel {e_lse:.2e}, row_loss rel {e_rl:.2e}, dH rel L2 {e_dh:.2e}")
    assert e_lse <= LOSS_RTOL and e_rl <= LOSS_RTOL and e_dh <= GRAD_RTOL
    rl_all = row_loss.double().cpu().numpy()
    want = float((w.astype(np.float64) * rl_all).sum() / w.astype(np.float64).sum())
    e_loss = abs(float(loss.item()) - want) / abs(want)
    col = dW.double().sum(dim=0)
    e_col = float(col.norm() / dW.double().norm())
    say(f"  loss vs weighted mean of row losses rel {e_loss:.2e}; |sum_v dW[v,:]| / |dW| {e_col:.2e}")
    assert e_loss <= 1e-5 and e_col <= 1e-2
