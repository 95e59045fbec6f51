"""The debug aids on the GPU: KD_VALIDATE=1 rejects a cache with an id
outside [0, V) before any other work, and leaves valid calls' results
unchanged; the debug build (device-side bounds checks on the cache-entry
scatters and gathers) passes its checks and gives bit-identical results to
the release build."""
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


def _inputs(name="tiny", **kw):
    cfg = get_config(name, **kw)
    return cfg, make_inputs(cfg, seed=3)


def _fwd_bwd(kd, H, W, idx, t, T, chunk, labels=None, weights=None):
    import torch
    if labels is None and weights is None:
        loss, lse, row_kl = kd.forward(H, W, idx, t, T, chunk, want_row_kl=True)
        dH, dW = kd.backward(H, W, idx, t, lse, None, T, chunk)
    else:
        kw = dict(row_weight=weights, labels=labels, kd_weight=0.5, ce_weight=0.5, scale_T2=True)
        loss, lse, row_kl = kd.forward_ex(H, W, idx, t, T, chunk, want_row_loss=True, **kw)
        dH, dW = kd.backward_ex(H, W, idx, t, lse, None, T, chunk, **kw)
    torch.cuda.synchronize()
    return [x.detach().clone() for x in (loss, lse, row_kl, dH, dW)]


def _bitwise_equal(a, b):
    import torch
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_validate_env_rejects_out_of_range_ids(monkeypatch):
    import torch
    import lm_head_top_amd as kd
    cfg, inp = _inputs()
    H, W, idx, t = to_device(inp)
    bad = idx.clone()
    bad[cfg.N // 2, 3] = cfg.V  # one id past the vocabulary
    say(f"KD_VALIDATE=1 with an id = V: N={cfg.N} V={cfg.V}")
    monkeypatch.setenv("KD_VALIDATE", "1")
    with pytest.raises(kd.KDError) as e:
        kd.forward(H, W, bad, t, 1.0, cfg.chunk)
    assert e.value.status == 5
    loss, lse = kd.forward(H, W, idx, t, 1.0, cfg.chunk)
    with pytest.raises(kd.KDError) as e:
        kd.backward(H, W, bad, t, lse, None, 1.0, cfg.chunk)
    assert e.value.status == 5
    with pytest.raises(kd.KDError) as e:
        kd.forward_noalloc(H, W, bad, t, 1.0, cfg.chunk)
    assert e.value.status == 5
    neg = idx.clone()
    neg[0, 0] = -1
    with pytest.raises(kd.KDError) as e:
        kd.forward_keep(H, W, neg, t, 1.0, cfg.chunk)
    assert e.value.status == 5
    # without the variable the same call runs (out-of-range ids are dropped)
    monkeypatch.delenv("KD_VALIDATE")
    loss, _ = kd.forward(H, W, bad, t, 1.0, cfg.chunk)
    torch.cuda.synchronize()
    assert np.isfinite(loss.item())


def test_validate_env_leaves_valid_results_unchanged(monkeypatch):
    import lm_head_top_amd as kd
    cfg, inp = _inputs()
    H, W, idx, t = to_device(inp)
    monkeypatch.delenv("KD_VALIDATE", raising=False)
    plain = _fwd_bwd(kd, H, W, idx, t, 2.0, cfg.chunk)
    monkeypatch.setenv("KD_VALIDATE", "1")
    checked = _fwd_bwd(kd, H, W, idx, t, 2.0, cfg.chunk)
    say(f"KD_VALIDATE=1 on valid ids: loss {plain[0].item():.7g} / {checked[0].item():.7g}")
    _bitwise_equal(plain, checked)


@pytest.mark.parametrize("case", ["tiny", "ragged_ext"])
def test_debug_build_passes_its_checks_and_matches_release(case):
    import torch
    import lm_head_top_amd as kd
    import os
    if not os.path.exists(kd.debug_lib_path()):
        pytest.skip("libkdtopk_debug.so not built")
    if case == "tiny":
        cfg, inp = _inputs()
        labels = weights = None
    else:
        # vocab tail tile, D tail, ragged last chunk, labels and weights
        cfg, inp = _inputs("tiny", N=700, D=200, V=4264, K=24, chunk=192)
        rng = np.random.default_rng(5)
        y = rng.integers(0, cfg.V, cfg.N).astype(np.int32)
        y[rng.random(cfg.N) < 0.1] = -1
        labels = torch.from_numpy(y).cuda()
        weights = torch.from_numpy((rng.random(cfg.N) > 0.2).astype(np.float32)).cuda()
    H, W, idx, t = to_device(inp)
    say(f"debug build: {case} N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk}")
    release = _fwd_bwd(kd, H, W, idx, t, 1.0, cfg.chunk, labels, weights)
    prev = kd.swap_library(kd.debug_lib_path())
    try:
        debug = _fwd_bwd(kd, H, W, idx, t, 1.0, cfg.chunk, labels, weights)  # raises on a failed check
    finally:
        kd.swap_library(prev)
    _bitwise_equal(release, debug)
