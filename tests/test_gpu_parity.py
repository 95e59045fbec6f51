"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bars: loss, lse and per-row KL within relative 1e-3; dH and dW within relative
L2 1e-2; cache-id handling exact (sign-pattern probe).
"""
import math

import numpy as np
import pytest

from oracle import kl_oracle as O
from synth import KDConfig, f32_to_bf16_bits, get_config, make_inputs
from tests.kdcase import assert_parity, rel, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()  # raises if the HIP library is missing: no fallback
    torch.cuda.set_device(0)


def _oracle(inp, T, grad_loss=1.0):
    f = O.forward(inp["H"], inp["W"], inp["idx"], inp["t"], T)
    b = O.backward(inp["H"], inp["W"], inp["idx"], inp["t"], T, grad_loss=grad_loss)
    return {**f, **b}


def _case(cfg, seed=0):
    say(f"case {cfg.name} N={cfg.N} D={cfg.D} V={cfg.V} K={cfg.K} chunk={cfg.chunk} "
        f"T={cfg.T} ids={cfg.ids} seed={seed}")
    return make_inputs(cfg, seed)


def test_tiny_config():
    cfg = get_config("tiny")
    inp = _case(cfg)
    assert_parity(run_gpu(inp, cfg.T, cfg.chunk), _oracle(inp, cfg.T), what="tiny")


def test_ragged_multi_tile():
    # vocab tail tile (5000 = 19*256 + 136), D tail (200 = 256 - 56), ragged last chunk
    cfg = KDConfig("ragged", N=700, D=200, V=5000, K=37, chunk=256, cfg_id=11)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.0, cfg.chunk), _oracle(inp, 1.0), what="ragged")


def test_temperature_and_grad_scale():
    cfg = get_config("tiny").replace(name="tiny_T2", T=2.0, cfg_id=12)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 2.0, cfg.chunk, grad_loss=0.37), _oracle(inp, 2.0, 0.37),
                  what="T=2")


def test_low_temperature():
    """T = 0.25 sharpens both distributions (student logits up to ~16 in
    magnitude, teacher mass on few ids)."""
    cfg = get_config("tiny").replace(name="tiny_T025", T=0.25, cfg_id=24)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 0.25, cfg.chunk), _oracle(inp, 0.25), what="T=0.25")


def test_chunk_larger_than_N_and_not_tile_multiple():
    cfg = KDConfig("clamp", N=300, D=64, V=1000, K=9, chunk=100000, ids="uniform", cfg_id=13)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.0, cfg.chunk), _oracle(inp, 1.0), what="clamp")
    cfg2 = cfg.replace(chunk=77)
    assert_parity(run_gpu(inp, 1.0, cfg2.chunk), _oracle(inp, 1.0), what="chunk77")


def test_chunk_independence():
    cfg = get_config("tiny")
    inp = _case(cfg)
    a = run_gpu(inp, 1.0, 64)
    b = run_gpu(inp, 1.0, 256)
    assert abs(a["loss"] - b["loss"]) <= 1e-6 * abs(b["loss"])
    assert np.max(np.abs(a["lse"] - b["lse"])) <= 1e-5
    assert rel(a["dH"], b["dH"]) <= 1e-2 and rel(a["dW"], b["dW"]) <= 1e-4


@pytest.mark.parametrize("N,chunk", [(2600, 128), (9000, 1024)])
def test_group_boundaries(N, chunk):
    """The backward keeps the G rows of up to 8 chunks (8192 positions) for one
    dW GEMM and runs dH over them in blocks of at most 4096 rows.  (2600, 128):
    three groups of 8 chunks, the last one ragged down to a 40-row chunk;
    (9000, 1024): a full group whose dH runs as two 4096-row blocks, then a
    ragged 808-row group."""
    cfg = KDConfig("groups", N=N, D=64, V=3000, K=16, chunk=chunk, ids="uniform", cfg_id=13)
    say(f"case group boundaries: N={N} chunk={chunk}")
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.0, chunk, grad_loss=0.6),
                  O.forward_backward_blocked(inp["H"], inp["W"], inp["idx"], inp["t"], 1.0, block=chunk,
                                             grad_loss=0.6), what=f"groups N={N} chunk={chunk}")


def test_deterministic_bitwise():
    cfg = KDConfig("det", N=600, D=256, V=3000, K=20, chunk=256, cfg_id=14)
    inp = _case(cfg)
    a = run_gpu(inp, 1.0, cfg.chunk)
    b = run_gpu(inp, 1.0, cfg.chunk)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_kl", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


def _edge_ids(V, K, N, seed):
    """Rows of K distinct ids that cover 0, V-1, every tile boundary +-1 and
    the tail tile, plus random fill."""
    edges = {0, 1, V - 1, V - 2}
    ntiles = (V + 255) // 256
    # boundaries of the first tiles, a spread of middle tiles and the last tiles
    for tb in sorted(set(list(range(1, 5)) + list(range(5, ntiles, 97)) +
                         list(range(max(1, ntiles - 4), ntiles)))):
        b = tb * 256
        edges.update({b - 1, b, b + 1})
    tail0 = (V - 1) // 256 * 256
    edges.update(range(tail0, min(V, tail0 + 8)))
    edges = sorted(e for e in edges if 0 <= e < V)
    r = np.random.default_rng(seed)
    rows = []
    pos = 0
    for _ in range(N):
        row = []
        while len(row) < K // 2:
            e = edges[pos % len(edges)]
            pos += 1
            if e not in row:
                row.append(e)
        while len(row) < K:
            x = int(r.integers(V))
            if x not in row:
                row.append(x)
        rows.append(row)
    return np.array(rows, dtype=np.int32), edges


@pytest.mark.parametrize("V", [4096 + 128 + 40, 201088])
def test_identity_probe_index_handling_is_exact(V):
    """H = I (N = D = 128), uniform teacher (p = 1/K), small W (q ~ 1/V << 1/K):
    dW = G^T exactly, so {(n, v): dW[v, n] < 0} must equal {(n, idx[n, k])}."""
    N = D = 128
    K = 16
    say(f"case identity probe V={V}")
    idx, edges = _edge_ids(V, K, N, 5)
    covered = set(idx.ravel().tolist())
    assert set(edges) <= covered
    H = f32_to_bf16_bits(np.eye(N, D, dtype=np.float32))
    r = np.random.default_rng(6)
    W = f32_to_bf16_bits((r.standard_normal((V, D)) * 1e-3).astype(np.float32))
    t = np.zeros((N, K), dtype=np.float32)
    inp = {"H": H, "W": W, "idx": idx, "t": t}
    g = run_gpu(inp, 1.0, 64)
    neg = g["dW"][:, :N].T < 0  # [n, v]
    want = np.zeros((N, V), dtype=bool)
    np.put_along_axis(want, idx.astype(np.int64), True, axis=1)
    assert np.array_equal(neg, want)
    # and the positive part is the student softmax everywhere else
    assert np.all(g["dW"][:, :N].T[~want] > 0)
    ref = O.forward(H, W, idx, t, 1.0)
    assert np.max(np.abs(g["row_kl"] - ref["row_kl"])) <= 1e-4 * np.max(np.abs(ref["row_kl"]))


def test_forward_gather_at_edge_ids():
    """Large logits (z ~ N(0, 9)) make a wrong gathered id visible in KL."""
    N, D, V, K = 96, 64, 201088, 24
    say("case gather edges")
    idx, _ = _edge_ids(V, K, N, 7)
    r = np.random.default_rng(8)
    H = f32_to_bf16_bits(r.standard_normal((N, D)).astype(np.float32))
    W = f32_to_bf16_bits((r.standard_normal((V, D)) * 3 / math.sqrt(D)).astype(np.float32))
    t = -np.sort(-r.standard_normal((N, K)).astype(np.float32) * 2, axis=1)
    inp = {"H": H, "W": W, "idx": idx, "t": t}
    g = run_gpu(inp, 1.0, 32, want_grads=True)
    ref = _oracle(inp, 1.0)
    assert np.max(np.abs(g["row_kl"] - ref["row_kl"]) / np.abs(ref["row_kl"])) <= 1e-4
    assert_parity(g, ref, what="gather-edges")


def test_max_vocabulary():
    """V = KD_MAX_V, the largest vocabulary accepted: 4096 vocab tiles, so the
    bucketing runs with its fewest counters per tile, and ids reach the last
    tile.  Two chunks, the second ragged; fp64 oracle row-blocked by chunk."""
    N, D, K, chunk = 300, 64, 40, 256
    V = 1 << 20
    say(f"case max vocabulary N={N} D={D} V={V} K={K} chunk={chunk}")
    idx, _ = _edge_ids(V, K, N, 21)
    r = np.random.default_rng(22)
    H = f32_to_bf16_bits(r.standard_normal((N, D)).astype(np.float32))
    W = f32_to_bf16_bits((r.standard_normal((V, D)) / math.sqrt(D)).astype(np.float32))
    t = -np.sort(-r.standard_normal((N, K)).astype(np.float32) * math.sqrt(3), axis=1)
    inp = {"H": H, "W": W, "idx": idx, "t": t}
    g = run_gpu(inp, 1.0, chunk)
    ref = O.forward_backward_blocked(H, W, idx, t, 1.0, block=chunk)
    assert_parity(g, ref, what="V=KD_MAX_V")


def test_k1_and_k_equals_v():
    cfg = KDConfig("k1", N=130, D=64, V=1000, K=1, chunk=64, ids="uniform", cfg_id=15)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.0, cfg.chunk), _oracle(inp, 1.0), what="K=1")
    cfg = KDConfig("kV", N=70, D=32, V=200, K=200, chunk=64, ids="uniform", cfg_id=16)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.5, cfg.chunk), _oracle(inp, 1.5), what="K=V")


def test_max_k():
    cfg = KDConfig("kmax", N=100, D=64, V=3000, K=256, chunk=64, ids="uniform", cfg_id=17)
    inp = _case(cfg)
    assert_parity(run_gpu(inp, 1.0, cfg.chunk), _oracle(inp, 1.0), what="K=256")


def test_minus_inf_teacher_logits():
    """Cache entries with teacher logit -inf (a masked token) get p = 0 and
    add nothing (0 log 0 = 0); rows with a single finite entry put all their
    mass on one id."""
    cfg = KDConfig("neginf", N=200, D=64, V=3000, K=32, chunk=64, ids="uniform", cfg_id=23)
    inp = _case(cfg)
    inp["t"][0::2, 20:] = -np.inf
    inp["t"][1::4, 1:] = -np.inf
    g = run_gpu(inp, 1.0, cfg.chunk)
    ref = _oracle(inp, 1.0)
    assert np.all(np.isfinite(g["row_kl"]))
    assert_parity(g, ref, what="-inf teacher logits")


def test_duplicate_ids_scatter_add():
    cfg = KDConfig("dup", N=64, D=32, V=500, K=8, chunk=32, ids="uniform", cfg_id=18)
    inp = _case(cfg)
    inp["idx"][:, 1] = inp["idx"][:, 0]
    inp["idx"][5, 2:5] = inp["idx"][5, 0]
    assert_parity(run_gpu(inp, 1.0, cfg.chunk), _oracle(inp, 1.0), what="dup")


def test_validate_flags():
    import torch
    import lm_head_top_amd as kd
    idx = torch.tensor([[0, 1, 2], [3, 4, 5]], dtype=torch.int32, device="cuda")
    assert kd.validate(idx, 6) == 0
    assert kd.validate(idx, 5) == 1
    idx[1, 2] = 3
    assert kd.validate(idx, 6) == 2
    idx[0, 0] = -1
    assert kd.validate(idx, 6) == 3


def test_empty_batch():
    import torch
    import lm_head_top_amd as kd
    say("case empty batch")
    H = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((10, 16), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((0, 3), dtype=torch.int32, device="cuda")
    t = torch.zeros((0, 3), dtype=torch.float32, device="cuda")
    loss, lse = kd.forward(H, W, idx, t, 1.0, 8)
    assert loss.item() == 0.0 and lse.numel() == 0
    dW0 = torch.full((10, 16), 2.5, dtype=torch.float32, device="cuda")
    dH, dW = kd.backward(H, W, idx, t, lse, None, 1.0, 8, dW=dW0.clone())
    assert torch.equal(dW, dW0) and dH.numel() == 0


def test_dw_accumulates_into_caller_buffer():
    import torch
    import lm_head_top_amd as kd
    cfg = KDConfig("acc", N=200, D=64, V=700, K=10, chunk=64, ids="uniform", cfg_id=19)
    inp = _case(cfg)
    H, W, idx, t = to_device(inp)
    _, lse = kd.forward(H, W, idx, t, 1.0, cfg.chunk)
    r = np.random.default_rng(3).standard_normal((cfg.V, cfg.D)).astype(np.float32)
    dW_in = torch.from_numpy(r).cuda()
    _, dW = kd.backward(H, W, idx, t, lse, None, 1.0, cfg.chunk, dW=dW_in.clone())
    ref = O.backward(inp["H"], inp["W"], inp["idx"], inp["t"], 1.0, dW_in=r)
    assert rel(dW.double().cpu().numpy(), ref["dW"]) <= 1e-2
    assert rel(dW.double().cpu().numpy() - r, ref["dW"] - r) <= 1e-2


def test_autograd_function_matches_entry_points():
    import torch
    import lm_head_top_amd as kd
    cfg = KDConfig("ag", N=150, D=96, V=900, K=12, chunk=64, ids="uniform", cfg_id=20)
    inp = _case(cfg)
    H, W, idx, t = to_device(inp)
    Hr = H.clone().requires_grad_(True)
    Wr = W.clone().requires_grad_(True)
    loss = kd.KDTopKKL.apply(Hr, Wr, idx, t, 1.0, cfg.chunk)
    (2.0 * loss).backward()
    ref = _oracle(inp, 1.0, grad_loss=2.0)
    assert abs(loss.item() - ref["loss"]) <= 1e-3 * ref["loss"]
    from tests.kdcase import bf16_tensor_to_f64
    assert rel(bf16_tensor_to_f64(Hr.grad), ref["dH"]) <= 1e-2
    assert rel(bf16_tensor_to_f64(Wr.grad), ref["dW"]) <= 1e-2


def test_invalid_ids_are_memory_safe():
    """Out-of-range ids give unspecified values but no fault, and validate flags them."""
    import torch
    import lm_head_top_amd as kd
    cfg = KDConfig("bad", N=64, D=32, V=300, K=6, chunk=32, ids="uniform", cfg_id=21)
    inp = _case(cfg)
    inp["idx"][3, 2] = 300
    inp["idx"][7, 0] = -5
    inp["idx"][9, 1] = 1 << 30
    H, W, idx, t = to_device(inp)
    assert kd.validate(idx, cfg.V) & 1
    loss, lse = kd.forward(H, W, idx, t, 1.0, cfg.chunk)
    dH, dW = kd.backward(H, W, idx, t, lse, None, 1.0, cfg.chunk)
    torch.cuda.synchronize()
    # rows without bad ids are still right
    ref = O.rows_forward(inp["H"], inp["W"], inp["idx"], inp["t"], [0, 1, 20], cfg.N, 1.0)
    assert np.allclose(lse.double().cpu().numpy()[[0, 1, 20]], ref["lse"], rtol=1e-4)


def test_concurrent_streams_with_distinct_workspaces():
    """Two problems on two streams at once (default priority), each with its
    own workspace: results bitwise equal to each problem run alone."""
    import torch
    import lm_head_top_amd as kd
    cfgs = [KDConfig("s1", N=1500, D=256, V=9000, K=32, chunk=512, ids="uniform", cfg_id=21),
            KDConfig("s2", N=900, D=192, V=7000, K=20, chunk=256, ids="uniform", cfg_id=22)]
    say("case concurrent streams")
    tens = [to_device(make_inputs(c, 1)) for c in cfgs]

    def run(i, ws):
        H, W, idx, t = tens[i]
        c = cfgs[i]
        loss, lse = kd.forward(H, W, idx, t, 1.0, c.chunk, workspace=ws)
        dH, dW = kd.backward(H, W, idx, t, lse, None, 1.0, c.chunk, workspace=ws)
        return loss, lse, dH, dW

    wss = [torch.empty(kd.workspace_size(c.N, c.D, c.V, c.K, c.chunk), dtype=torch.uint8, device="cuda")
           for c in cfgs]
    alone = [run(i, wss[i]) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    together = [None, None]
    for _ in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                together[i] = run(i, wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(alone[i], together[i]):
                assert torch.equal(a, b)
