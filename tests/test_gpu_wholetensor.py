"""Whole-tensor gradient parity at LM-head widths: every element of dH and dW
against the fp64 oracle, relative L2 within 1e-2.

* A D tail and several D tiles (D = 584 = 2 x 256 + 72): dH and dW tiles with
  a non-zero column-tile index, the partial last D tile, the banded tile orders
  with more than one column tile, and dH split over the vocabulary with its
  reduce kernel (a group of 1100 rows has too few tiles to fill the device).
* The toy LM head (8192 x 4096 x 131072, chunk 1024) whole, in the launch
  configuration the benchmark times; the oracle runs row-blocked in the test.
* A group of chunks whose G rows exceed 32-bit buffer offsets (V = 2^20, 2560
  rows of G = 5 GiB), so dH and dW run in two row blocks each.
"""
import numpy as np
import pytest

from oracle import kl_oracle as O
from synth import get_config, make_inputs
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


def _run_and_compare(inp, T, chunk, block, what):
    import torch
    import lm_head_top_amd as kd
    H, W, idx, t = to_device(inp)
    loss, lse, row_kl = kd.forward(H, W, idx, t, T, chunk, want_row_kl=True)
    dH, dW = kd.backward(H, W, idx, t, lse, None, T, chunk)
    torch.cuda.synchronize()
    g_loss = float(loss.item())
    g_lse = lse.double().cpu().numpy()
    g_dh = bf16_tensor_to_f64(dH)
    g_dw = dW.double().cpu().numpy()
    del H, W, idx, t, dH, dW, lse, row_kl, loss
    torch.cuda.empty_cache()
    say(f"  {what}: GPU done, running the row-blocked oracle (block {block})")
    ref = O.forward_backward_blocked(inp["H"], inp["W"], inp["idx"], inp["t"], T, block=block)
    lr = abs(g_loss - ref["loss"]) / abs(ref["loss"])
    e_lse = float(np.max(np.abs(g_lse - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0)))
    eh, ew = rel(g_dh, ref["dH"]), rel(g_dw, ref["dW"])
    # the worst vocabulary row and hidden column of dW, relative to the whole tensor's norm
    nw = np.linalg.norm(ref["dW"])
    row_err = float(np.max(np.linalg.norm(g_dw - ref["dW"], axis=1)) / nw)
    say(f"  {what}: loss rel {lr:.2e}, lse {e_lse:.2e}, dH rel L2 {eh:.2e}, dW rel L2 {ew:.2e} "
        f"(worst dW row {row_err:.2e} of the norm)")
    assert lr <= LOSS_RTOL and e_lse <= LOSS_RTOL
    assert eh <= GRAD_RTOL and ew <= GRAD_RTOL


def test_whole_grads_with_d_tail_and_several_d_tiles():
    cfg = get_config("toy").replace(name="dtail", N=1100, D=584, V=5000, K=16, chunk=256)
    say(f"case whole-tensor N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} (zipf ids)")
    _run_and_compare(make_inputs(cfg, 3), cfg.T, cfg.chunk, 1100, "D tail")


def test_whole_grads_toy_lm_head():
    cfg = get_config("toy")
    say(f"case whole-tensor toy N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk}")
    _run_and_compare(make_inputs(cfg, 0), cfg.T, cfg.chunk, 1024, "toy")


def test_whole_grads_when_g_rows_exceed_32bit_offsets():
    cfg = get_config("toy").replace(name="bigv", N=2560, D=64, V=1 << 20, K=8, chunk=2560)
    say(f"case whole-tensor N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} "
        "(G block of 5 GiB: two row blocks per gradient GEMM)")
    _run_and_compare(make_inputs(cfg, 5), cfg.T, cfg.chunk, 256, "split")
