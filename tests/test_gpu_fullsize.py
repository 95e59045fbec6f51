"""Full-size workloads in the launch configuration the benchmark times.

The oracle cannot redo a whole problem of this size on the host in a test, so
the checks are (a) sampled rows, which the oracle computes one by one (lse,
KL_n and the dH row only need that row's logits), (b) properties that hold at
any size (the loss is the mean of the per-row KL; every row of G sums to zero,
so the columns of dW sum to zero), (c) where tests/golden holds the oracle's
full-problem results for the workload (written by tests/golden/make_golden.py,
which runs only the oracle), the whole loss, lse and KL_n vectors and sampled
dW rows, and (d) peak memory linear in N.
"""
import json
import os

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


def _sample_rows(N, n=6, seed=0):
    r = np.random.default_rng(seed)
    rows = set([0, N - 1]) | set(r.integers(0, N, n - 2).tolist())
    return sorted(rows)


@pytest.mark.parametrize("name", ["toy", "large_vocab", "long", "very_long"])
def test_full_size_sampled_rows(name):
    import torch
    import lm_head_top_amd as kd
    cfg = get_config(name)
    say(f"case full-size {name}: N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk}")
    inp = make_inputs(cfg, 0)
    H, W, idx, t = to_device(inp)
    loss, lse, row_kl = kd.forward(H, W, idx, t, cfg.T, cfg.chunk, want_row_kl=True)
    dH, dW = kd.backward(H, W, idx, t, lse, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.N)
    ref = O.rows_forward(inp["H"], inp["W"], inp["idx"], inp["t"], rows, cfg.N, cfg.T)
    g_lse = lse.double().cpu().numpy()[rows]
    g_kl = row_kl.double().cpu().numpy()[rows]
    g_dh = bf16_tensor_to_f64(dH[rows])
    e_lse = np.max(np.abs(g_lse - ref["lse"]) / np.abs(ref["lse"]))
    e_kl = np.max(np.abs(g_kl - ref["row_kl"]) / np.abs(ref["row_kl"]))
    e_dh = rel(g_dh, ref["dH"])
    say(f"  rows {rows}: lse rel {e_lse:.2e}, row_kl rel {e_kl:.2e}, dH rel L2 {e_dh:.2e}")
    assert e_lse <= LOSS_RTOL and e_kl <= LOSS_RTOL and e_dh <= GRAD_RTOL
    # loss is the mean over all N rows of KL_n
    mean_kl = row_kl.double().mean().item()
    assert abs(loss.item() - mean_kl) <= 1e-6 * abs(mean_kl)
    assert np.isfinite(row_kl.cpu().numpy()).all() and (row_kl.cpu().numpy() > 0).all()
    # sum_v dW[v, :] = sum_n (sum_v G[n, v]) H[n, :] = 0 up to rounding of G to bf16
    colsum = dW.double().sum(dim=0)
    scale = dW.double().abs().sum(dim=0)
    worst = (colsum.abs() / scale).max().item()
    say(f"  dW column sums: worst |sum| / sum|.| = {worst:.2e}")
    assert worst <= 1e-2
    assert torch.isfinite(dW).all().item() and torch.isfinite(dH.float()).all().item()
    _check_golden(name, loss, lse, row_kl, dW)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _check_golden(name, loss, lse, row_kl, dW):
    path = os.path.join(GOLDEN, f"{name}_seed0.npz")
    if not os.path.exists(path):
        say(f"  no oracle golden file for {name}; sampled rows and properties only")
        return
    import torch
    g = np.load(path)  # plain arrays, allow_pickle stays False
    meta = json.loads(str(g["meta"]))
    cfg = get_config(name)
    assert (meta["N"], meta["D"], meta["V"], meta["K"]) == (cfg.N, cfg.D, cfg.V, cfg.K)
    e_loss = abs(loss.item() - float(g["loss"])) / abs(float(g["loss"]))
    e_lse = np.max(np.abs(lse.double().cpu().numpy() - g["lse"]) / np.abs(g["lse"].astype(np.float64)))
    kl_ref = g["row_kl"].astype(np.float64)
    e_kl = np.max(np.abs(row_kl.double().cpu().numpy() - kl_ref) / np.abs(kl_ref))
    rows = torch.from_numpy(g["dw_rows"]).to(dW.device)
    got = dW.index_select(0, rows).double().cpu().numpy()
    e_dw = max(rel(got[i], g["dw"][i]) for i in range(got.shape[0]))
    say(f"  golden: loss rel {e_loss:.2e}, all-rows lse rel {e_lse:.2e}, row_kl rel {e_kl:.2e}, "
        f"dW rows {g['dw_rows'].tolist()} worst rel L2 {e_dw:.2e}")
    assert e_loss <= LOSS_RTOL and e_lse <= LOSS_RTOL and e_kl <= LOSS_RTOL
    assert e_dw <= GRAD_RTOL


def test_peak_memory_linear_in_N():
    """Peak device memory of one forward + backward grows linearly in N with a
    slope of about H + dH + the cache + lse per position (no N x V term).  The
    N start where the backward's group of chunks (8192 positions) is full;
    below that the workspace is smaller still."""
    import torch
    import lm_head_top_amd as kd
    D, V, K, chunk = 4096, 131072, 100, 2048
    peaks = []
    Ns = [8192, 16384, 32768]
    W = torch.zeros((V, D), dtype=torch.bfloat16, device="cuda")
    for N in Ns:
        say(f"case peak memory N={N}")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        H = torch.randn((N, D), device="cuda", dtype=torch.bfloat16)
        idx = torch.randint(0, V, (N, K), device="cuda", dtype=torch.int32)
        t = torch.randn((N, K), device="cuda")
        loss, lse = kd.forward(H, W, idx, t, 1.0, chunk)
        dH, dW = kd.backward(H, W, idx, t, lse, None, 1.0, chunk)
        torch.cuda.synchronize()
        peaks.append(torch.cuda.max_memory_allocated() - base)
        del H, idx, t, loss, lse, dH, dW
    slope = (peaks[2] - peaks[0]) / (Ns[2] - Ns[0])
    mid = peaks[0] + slope * (Ns[1] - Ns[0])
    say(f"  peaks {[round(p / 2**30, 3) for p in peaks]} GiB; slope {slope / 1024:.2f} KiB/token")
    assert abs(peaks[1] - mid) <= 0.02 * peaks[1]           # linear
    assert slope <= 1.25 * (4 * D + 8 * K + 8)               # ~16.8 KiB per position
    assert peaks[2] < 8 * 2**30                              # far below one N x V fp32 grid
