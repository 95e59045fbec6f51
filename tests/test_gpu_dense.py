"""Dense-teacher (online) mode: KL over the full vocabulary against the same
fp64 oracle with every token id as a cache entry (its K = V case, which the
oracle pins check against scipy's rel_entr and torch's kl_div)."""
import numpy as np
import pytest

from oracle import kl_oracle as O
from synth import get_config, make_inputs
from synth.inputs import KDConfig, f32_to_bf16_bits, bf16_bits_to_f32
from tests.kdcase import GRAD_RTOL, LOSS_RTOL, assert_parity, bf16_tensor_to_f64, rel, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def _teacher(N, V, seed, bf16):
    t = (np.random.default_rng(seed).standard_normal((N, V)) * 3 ** 0.5).astype(np.float32)
    if bf16:
        bits = f32_to_bf16_bits(t)
        return bits, bf16_bits_to_f32(bits)
    return t, t


def _run(inp, teacher, bf16, T, chunk, grad_loss=None):
    import torch
    import lm_head_top_amd as kd
    H, W, _, _ = to_device(inp)
    if bf16:
        tt = torch.from_numpy(teacher.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        tt = torch.from_numpy(teacher).cuda()
    loss, lse, lse_t, row_kl = kd.dense_forward(H, W, tt, T, chunk, want_row_kl=True)
    g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    dH, dW = kd.dense_backward(H, W, tt, lse, lse_t, g, T, chunk)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
            "row_kl": row_kl.double().cpu().numpy(), "dH": bf16_tensor_to_f64(dH),
            "dW": dW.double().cpu().numpy(), "lse_t": lse_t.double().cpu().numpy()}


@pytest.mark.parametrize("case", ["tiny_f32", "tiny_bf16", "ragged_T2"])
def test_dense_matches_oracle(case):
    if case.startswith("tiny"):
        cfg, T, g = get_config("tiny"), 1.0, None
    else:
        cfg = KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, T=2.0, ids="uniform", cfg_id=7)
        T, g = 2.0, 0.37
    bf16 = case.endswith("bf16")
    say(f"case dense {case}: N={cfg.N} D={cfg.D} V={cfg.V} chunk={cfg.chunk} T={T}")
    inp = make_inputs(cfg, 9)
    tdev, tf32 = _teacher(cfg.N, cfg.V, 10, bf16)
    out = _run(inp, tdev, bf16, T, cfg.chunk, g)
    idx = np.tile(np.arange(cfg.V, dtype=np.int32), (cfg.N, 1))
    ref = O.forward_backward_blocked(inp["H"], inp["W"], idx, tf32, T, block=cfg.chunk,
                                     grad_loss=1.0 if g is None else g)
    assert_parity(out, ref, what=f"dense {case}")
    # the teacher's own log-normaliser
    a = tf32.astype(np.float64) / T
    m = a.max(axis=1)
    lse_t = m + np.log(np.exp(a - m[:, None]).sum(axis=1))
    assert np.max(np.abs(out["lse_t"] - lse_t) / np.abs(lse_t)) <= LOSS_RTOL


def test_dense_full_size_sampled_rows():
    """Toy LM head with a dense fp32 teacher [8192, 131072]: sampled rows
    against the oracle, the loss against the mean of the row KLs."""
    import torch
    import lm_head_top_amd as kd
    cfg = get_config("toy")
    say(f"case dense full size: N={cfg.N} D={cfg.D} V={cfg.V}")
    inp = make_inputs(cfg, 0)
    H, W, _, _ = to_device(inp)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    tt = torch.randn((cfg.N, cfg.V), generator=g, device="cuda") * 3 ** 0.5
    loss, lse, lse_t, row_kl = kd.dense_forward(H, W, tt, cfg.T, cfg.chunk, want_row_kl=True)
    dH, dW = kd.dense_backward(H, W, tt, lse, lse_t, None, cfg.T, cfg.chunk)
    torch.cuda.synchronize()
    rows = [0, 1, 777, 4095, 4096, cfg.N - 1]
    t_rows = tt[rows].cpu().numpy()
    idx = np.tile(np.arange(cfg.V, dtype=np.int32), (len(rows), 1))
    ref = O.rows_forward(inp["H"][rows], inp["W"], idx, t_rows, np.arange(len(rows)), cfg.N, cfg.T)
    e_lse = np.max(np.abs(lse.double().cpu().numpy()[rows] - ref["lse"]) / np.abs(ref["lse"]))
    e_kl = np.max(np.abs(row_kl.double().cpu().numpy()[rows] - ref["row_kl"]) / np.abs(ref["row_kl"]))
    e_dh = rel(bf16_tensor_to_f64(dH[rows]), ref["dH"])
    say(f"  rows {rows}: lse rel {e_lse:.2e}, row_kl rel {e_kl:.2e}, dH rel L2 {e_dh:.2e}")
    assert e_lse <= LOSS_RTOL and e_kl <= LOSS_RTOL and e_dh <= GRAD_RTOL
    assert abs(loss.item() - row_kl.double().mean().item()) <= 1e-6 * abs(loss.item())
    colsum = dW.double().sum(dim=0)
    assert (colsum.abs() / dW.double().abs().sum(dim=0)).max().item() <= 1e-2
