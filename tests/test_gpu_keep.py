"""The comparators that keep instead of recomputing: kept gradient (G kept
from the forward) and kept logits (every chunk's fp32 logits kept from the
forward; the pages' next-best variant).  Parity with the oracle on small
cases, and agreement with the recompute path at the toy LM head (same forward
kernels, so the loss and lse are bitwise equal; dH and dW differ only by the
rounding order of G at the cached ids and by the dW accumulation order)."""
import numpy as np
import pytest

from oracle import kl_oracle as O
from synth import get_config, make_inputs
from synth.inputs import KDConfig
from tests.kdcase import GRAD_RTOL, assert_parity, bf16_tensor_to_f64, rel, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def _run_keep(inp, T, chunk, grad_loss=None, dW0=None):
    import torch
    import lm_head_top_amd as kd
    H, W, idx, t = to_device(inp)
    loss, lse, row_kl, ws = kd.forward_keep(H, W, idx, t, T, chunk, want_row_kl=True)
    g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    dW = None if dW0 is None else torch.from_numpy(dW0.astype(np.float32)).cuda()
    dH, dW = kd.backward_keep(H, W, idx.shape[1], ws, g, T, chunk, dW=dW)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
            "row_kl": row_kl.double().cpu().numpy(), "dH": bf16_tensor_to_f64(dH),
            "dW": dW.double().cpu().numpy()}


@pytest.mark.parametrize("case", ["tiny", "ragged_T2"])
def test_keep_matches_oracle(case):
    if case == "tiny":
        cfg, T, g = get_config("tiny"), 1.0, None
    else:
        cfg = KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, T=2.0, ids="uniform", cfg_id=7)
        T, g = 2.0, 0.37
    say(f"case keep {case}: N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} T={T}")
    inp = make_inputs(cfg, 5)
    dW0 = np.random.default_rng(1).standard_normal((cfg.V, cfg.D)) * 1e-3
    out = _run_keep(inp, T, cfg.chunk, g, dW0)
    ref = O.forward_backward_blocked(inp["H"], inp["W"], inp["idx"], inp["t"], T, block=cfg.chunk,
                                     grad_loss=1.0 if g is None else g,
                                     dW_in=dW0.astype(np.float32).astype(np.float64))
    assert_parity(out, ref, what=f"keep {case}")


def test_keep_agrees_with_recompute_at_full_size():
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("toy")
    say(f"case keep vs recompute, toy: N={cfg.N} D={cfg.D} V={cfg.V}")
    inp = make_inputs(cfg, 0)
    H, W, idx, t = to_device(inp)
    loss_r, lse_r = kd.forward(H, W, idx, t, cfg.T, cfg.chunk)
    dH_r, dW_r = kd.backward(H, W, idx, t, lse_r, None, cfg.T, cfg.chunk)
    loss_k, lse_k, ws = kd.forward_keep(H, W, idx, t, cfg.T, cfg.chunk)
    dH_k, dW_k = kd.backward_keep(H, W, cfg.K, ws, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(loss_r, loss_k) and torch.equal(lse_r, lse_k)
    eh = rel(bf16_tensor_to_f64(dH_k), bf16_tensor_to_f64(dH_r))
    ew = float((dW_k.double() - dW_r.double()).norm() / dW_r.double().norm())
    say(f"  loss and lse bitwise equal; dH rel L2 {eh:.2e}, dW rel L2 {ew:.2e}")
    assert eh <= 1e-3 and ew <= 1e-3
    assert eh <= GRAD_RTOL


def _run_keep_logits(inp, T, chunk, grad_loss=None, dW0=None):
    import torch
    import lm_head_top_amd as kd
    H, W, idx, t = to_device(inp)
    loss, lse, row_kl, ws = kd.forward_keep_logits(H, W, idx, t, T, chunk, want_row_kl=True)
    g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    dW = None if dW0 is None else torch.from_numpy(dW0.astype(np.float32)).cuda()
    dH, dW = kd.backward_keep_logits(H, W, idx, t, lse, ws, g, T, chunk, dW=dW)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
            "row_kl": row_kl.double().cpu().numpy(), "dH": bf16_tensor_to_f64(dH),
            "dW": dW.double().cpu().numpy()}


@pytest.mark.parametrize("case", ["tiny", "ragged_T2"])
def test_keep_logits_matches_oracle(case):
    if case == "tiny":
        cfg, T, g = get_config("tiny"), 1.0, None
    else:
        cfg = KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, T=2.0, ids="uniform", cfg_id=7)
        T, g = 2.0, 0.37
    say(f"case keep-logits {case}: N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} T={T}")
    inp = make_inputs(cfg, 6)
    dW0 = np.random.default_rng(2).standard_normal((cfg.V, cfg.D)) * 1e-3
    out = _run_keep_logits(inp, T, cfg.chunk, g, dW0)
    ref = O.forward_backward_blocked(inp["H"], inp["W"], inp["idx"], inp["t"], T, block=cfg.chunk,
                                     grad_loss=1.0 if g is None else g,
                                     dW_in=dW0.astype(np.float32).astype(np.float64))
    assert_parity(out, ref, what=f"keep-logits {case}")


def test_keep_logits_agrees_with_recompute_at_full_size():
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("toy")
    say(f"case keep-logits vs recompute, toy: N={cfg.N} D={cfg.D} V={cfg.V}")
    inp = make_inputs(cfg, 0)
    H, W, idx, t = to_device(inp)
    loss_r, lse_r = kd.forward(H, W, idx, t, cfg.T, cfg.chunk)
    dH_r, dW_r = kd.backward(H, W, idx, t, lse_r, None, cfg.T, cfg.chunk)
    loss_k, lse_k, ws = kd.forward_keep_logits(H, W, idx, t, cfg.T, cfg.chunk)
    dH_k, dW_k = kd.backward_keep_logits(H, W, idx, t, lse_k, ws, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(loss_r, loss_k) and torch.equal(lse_r, lse_k)
    eh = rel(bf16_tensor_to_f64(dH_k), bf16_tensor_to_f64(dH_r))
    ew = float((dW_k.double() - dW_r.double()).norm() / dW_r.double().norm())
    say(f"  loss and lse bitwise equal; dH rel L2 {eh:.2e}, dW rel L2 {ew:.2e}")
    assert eh <= 1e-3 and ew <= 1e-3
