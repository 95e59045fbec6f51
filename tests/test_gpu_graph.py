"""The hot path captured into a HIP graph: the allocation-free forward and the
backward (with a caller workspace and dW), replayed several times with other
eager work and synchronisations between the replays; every replay must be
bitwise equal to the same calls run eagerly.  The release entry points enqueue
kernels only (no memset, copy or host synchronisation), which is what makes
them capturable."""
import numpy as np
import pytest

from synth import get_config, make_inputs
from tests.kdcase import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def test_forward_noalloc_and_backward_replay_bitwise(monkeypatch):
    import torch
    import lm_head_top_amd as kd
    monkeypatch.delenv("KD_VALIDATE", raising=False)
    # vocab tail tile, D tail, ragged last chunk, several chunk groups
    cfg = get_config("tiny", N=700, D=200, V=4264, K=24, chunk=192)
    inp = make_inputs(cfg, seed=11)
    H, W, idx, t = to_device(inp)
    T = 2.0
    N, D, V, K = cfg.N, cfg.D, cfg.V, cfg.K
    say(f"graph capture: N={N} D={D} V={V} K={K} chunk={cfg.chunk}")
    ws = torch.empty(kd.workspace_size(N, D, V, K, cfg.chunk), dtype=torch.uint8, device="cuda")

    def run(loss, lse, dW):
        dW.zero_()
        kd.forward_noalloc(H, W, idx, t, T, cfg.chunk, loss=loss, lse=lse)
        dH, _ = kd.backward(H, W, idx, t, lse, None, T, cfg.chunk, dW=dW, workspace=ws)
        return dH

    # eager reference (also the warm-up: the library looks up its device
    # scratch and the compute-unit count on the first call)
    loss_e = torch.empty(1, dtype=torch.float32, device="cuda")
    lse_e = torch.empty(N, dtype=torch.float32, device="cuda")
    dW_e = torch.empty((V, D), dtype=torch.float32, device="cuda")
    dH_e = run(loss_e, lse_e, dW_e)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (loss_e, lse_e, dH_e, dW_e)]

    loss_g = torch.empty(1, dtype=torch.float32, device="cuda")
    lse_g = torch.empty(N, dtype=torch.float32, device="cuda")
    dW_g = torch.empty((V, D), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(loss_g, lse_g, dW_g)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dH_g = run(loss_g, lse_g, dW_g)
    for rep in range(3):
        # other eager work and synchronisations between the replays
        a = torch.randn(512, 512, device="cuda")
        (a @ a).sum().item()
        loss_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        dH_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (loss_g, lse_g, dH_g, dW_g)
        for name, x, y in zip(("loss", "lse", "dH", "dW"), got, ref):
            same = torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
            assert same, f"replay {rep}: {name} differs from the eager result"
        say(f"  replay {rep}: loss {loss_g.item():.7g} bitwise equal to eager")
    assert np.isfinite(ref[0].item())
