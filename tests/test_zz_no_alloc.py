"""kd_topk_kl_forward_noalloc (the forward whose scratch is the library's own
device array) against kd_topk_kl_forward (caller workspace) through the C ABI:
two calls in a row on one GPU, the second with a smaller input, each equal to
the workspace forward bit for bit (same kernels, same scratch layout) and to
the fp64 oracle within the loss bar.  The second call reuses the array the
first one filled, so stale contents would show."""
import numpy as np
import pytest

from oracle import kl_oracle as O
from synth import get_config, make_inputs
from tests.kdcase import LOSS_RTOL, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def _one(cfg, seed):
    import torch
    import lm_head_top_amd as kd
    say(f"case noalloc N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} T={cfg.T} seed={seed}")
    inp = make_inputs(cfg, seed)
    H, W, idx, t = to_device(inp)
    dev = H.device
    # outputs allocated up front, so the call itself allocates nothing anywhere
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(cfg.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(cfg.N, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    kd.forward_noalloc(H, W, idx, t, cfg.T, cfg.chunk, loss=loss, lse=lse, row_kl=row_kl)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    ref_loss, ref_lse, ref_kl = kd.forward(H, W, idx, t, cfg.T, cfg.chunk, want_row_kl=True)
    torch.cuda.synchronize()
    assert torch.equal(loss, ref_loss) and torch.equal(lse, ref_lse) and torch.equal(row_kl, ref_kl)
    if cfg.N * cfg.V <= (1 << 26):
        o = O.forward(inp["H"], inp["W"], inp["idx"], inp["t"], cfg.T)
        lr = abs(loss.item() - o["loss"]) / abs(o["loss"])
        e_lse = float(np.max(np.abs(lse.double().cpu().numpy() - o["lse"]) / np.abs(o["lse"])))
        say(f"  oracle: loss rel {lr:.2e}, lse max rel {e_lse:.2e}")
        assert lr <= LOSS_RTOL and e_lse <= LOSS_RTOL
    return float(loss.item())


def test_noalloc_forward_matches_the_workspace_forward_twice():
    big = get_config("toy")                      # 10.8 MiB of forward scratch
    small = get_config("toy").replace(name="ragged", N=300, D=200, V=4264, K=16, chunk=128, T=2.0)
    _one(big, 0)
    _one(small, 1)


def test_noalloc_forward_rejects_problems_beyond_the_array():
    import torch
    import lm_head_top_amd as kd
    dev = torch.device("cuda:0")
    N, D, V, K = 32768, 64, 131072, 4
    H = torch.zeros(N, D, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, D, dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(N, K, dtype=torch.int32, device=dev)
    t = torch.zeros(N, K, dtype=torch.float32, device=dev)
    with pytest.raises(kd.KDError, match="workspace too small"):
        kd.forward_noalloc(H, W, idx, t, 1.0, 16384)   # 83 MiB of forward scratch
