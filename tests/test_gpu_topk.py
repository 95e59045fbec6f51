"""Parity of the HIP teacher top-K cache writer with the CPU oracle.

Ids and logits must match exactly (integer and selection work: the kernel and
the oracle compare the same fp32 / bf16 values).  Small cases cover every load
path (16-byte loads, element loads for ragged rows or unaligned bases, fp32 and
bf16), ties, constant rows, signed zeros, infinities and K at its limits; the
full-size cases check sampled rows against the oracle and every row against
properties that hold at any size.
"""
import numpy as np
import pytest

from oracle import topk_oracle as TO
from tests.kdcase import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_top_amd as kd
    kd.load_library()
    torch.cuda.set_device(0)


def _run(host, K, bf16=False, offset=0):
    """host: fp32 array [N, V] (or uint16 bf16 bits).  offset > 0 shifts the
    device base by that many elements (unaligned rows)."""
    import torch
    import lm_head_top_amd as kd
    if bf16:
        flat = np.concatenate([np.zeros(offset, np.uint16), host.ravel()])
        t = torch.from_numpy(flat.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        flat = np.concatenate([np.zeros(offset, np.float32), host.ravel()])
        t = torch.from_numpy(flat).cuda()
    x = t[offset:].view(host.shape)
    idx, val = kd.topk_select(x, K)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy().astype(np.float64)


def _check(host, K, **kw):
    gi, gv = _run(host, K, **kw)
    oi, ov = TO.topk_select(host, K)
    bad = np.nonzero((gi != oi).any(axis=1) | (gv != ov).any(axis=1))[0]
    say(f"  N={host.shape[0]} V={host.shape[1]} K={K} {kw}: {len(bad)} rows differ")
    assert len(bad) == 0, (bad[:5], gi[bad[0]][:10], oi[bad[0]][:10])


def _bf16(a):
    from synth import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(a, np.float32))


def test_random_rows_fp32_vector_path():
    say("case topk fp32 16-byte loads")
    r = np.random.default_rng(1)
    _check(r.standard_normal((64, 5000)).astype(np.float32) * 2, 100)


def test_tie_heavy_rows():
    say("case topk ties")
    r = np.random.default_rng(2)
    L = (r.integers(-6, 7, size=(48, 12288)) * 0.25).astype(np.float32)
    _check(L, 256)
    _check(L, 1)


def test_element_path_and_unaligned_base():
    say("case topk element loads")
    r = np.random.default_rng(3)
    _check(r.standard_normal((33, 1001)).astype(np.float32), 37)           # V % 4 != 0
    _check(r.standard_normal((17, 4096)).astype(np.float32), 50, offset=1)  # base not 16-byte aligned


def test_bf16_paths():
    say("case topk bf16")
    r = np.random.default_rng(4)
    _check(_bf16(r.standard_normal((40, 8200)) * 3), 100, bf16=True)      # 16-byte loads
    _check(_bf16(r.standard_normal((9, 1003))), 64, bf16=True)            # element loads
    _check(_bf16(np.round(r.standard_normal((12, 4096)) * 2) / 2), 200, bf16=True)  # ties


def test_special_values_and_limits():
    say("case topk special values")
    row = np.array([-1.0, -0.0, -np.inf, 0.0, np.inf, -0.0, 2.0, 0.5], dtype=np.float32)
    _check(np.tile(row, (3, 1)), 8)                                    # K = V, signed zeros, inf
    _check(np.full((5, 9000), 3.5, dtype=np.float32), 256)              # constant rows
    r = np.random.default_rng(5)
    _check(r.standard_normal((4, 256)).astype(np.float32), 256)         # K = V = 256
    _check(r.standard_normal((3, 20000)).astype(np.float32) - 1e3, 100)  # all negative


def test_very_long_rows():
    """Rows of 2^21 logits (16 times the toy vocabulary): many load batches
    and compactions per row, fp32 and bf16 (with a ragged tail)."""
    say("case topk very long rows")
    r = np.random.default_rng(6)
    _check(r.standard_normal((3, 1 << 21)).astype(np.float32), 256)
    _check(_bf16(r.standard_normal((2, (1 << 21) + 3))), 100, bf16=True)


@pytest.mark.parametrize("V,dt", [((0x7FFFFFF0 // 4), "f32"), ((1 << 31) - 1, "f32"), ((1 << 31) - 1, "bf16")])
def test_rows_at_the_index_limits(V, dt):
    """One row at the largest sizes: 2^31 - 16 bytes of fp32 (the last row
    the 16-byte path takes, its offsets at the top of 32 bits) and 2^31 - 1
    logits (the largest row accepted; the element path, ids up to 2^31 - 2).
    The row holds -5 everywhere and 8 planted larger values, so the result is
    known by construction: the planted values best first, then -5 at the
    lowest free ids."""
    import torch
    import lm_head_top_amd as kd
    K = 16
    say(f"case topk row at the index limit V={V} {dt}")
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    x = torch.full((1, V), -5.0, dtype=dtype, device="cuda")
    ids = [V - 1, V - 2, V - 5, V // 2, 123456789, 7, 3, 0]
    vals = [9.0, 8.5, 8.0, 7.0, 6.5, 6.0, 5.5, 5.0]
    x[0, torch.tensor(ids, device="cuda")] = torch.tensor(vals, dtype=dtype, device="cuda")
    idx, val = kd.topk_select(x, K)
    torch.cuda.synchronize()
    del x
    free = [i for i in range(K + len(ids)) if i not in ids][:K - len(ids)]
    want_i = ids + free
    want_v = vals + [-5.0] * len(free)
    assert idx[0].cpu().tolist() == want_i
    assert val[0].cpu().tolist() == want_v


def test_empty_batch():
    import torch
    import lm_head_top_amd as kd
    idx, val = kd.topk_select(torch.empty((0, 100), device="cuda"), 10)
    torch.cuda.synchronize()
    assert idx.shape == (0, 10) and val.shape == (0, 10)


@pytest.mark.parametrize("N,V,dt", [(8192, 131072, "f32"), (2048, 201088, "bf16")])
def test_full_size(N, V, dt):
    """Teacher logits of the toy LM head (fp32) and of the gpt-oss vocabulary
    (bf16), drawn on the device from a seeded generator: 24 sampled rows
    against the oracle, every row against the properties of a top-K."""
    import torch
    import lm_head_top_amd as kd
    K = 100
    say(f"case topk full size N={N} V={V} {dt}")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randn((N, V), generator=g, device="cuda") * 3 ** 0.5
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    idx, val = kd.topk_select(x, K)
    torch.cuda.synchronize()
    rows = sorted(set([0, N - 1] + np.random.default_rng(8).integers(0, N, 22).tolist()))
    sample = x[rows].contiguous()
    host = (sample.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16"
            else sample.cpu().numpy())
    oi, ov = TO.topk_select(host, K)
    assert (idx[rows].cpu().numpy() == oi).all()
    assert (val[rows].double().cpu().numpy() == ov).all()
    # every row: best first, ids distinct, values are the logits at the ids,
    # and no unselected logit beats the K-th
    xf = x.float()
    assert (val[:, 1:] <= val[:, :-1]).all().item()
    s, _ = torch.sort(idx, dim=1)
    assert (s[:, 1:] != s[:, :-1]).all().item()
    assert torch.equal(torch.gather(xf, 1, idx.long()), val)
    rest = xf.scatter(1, idx.long(), float("-inf"))
    assert (rest.max(dim=1).values <= val[:, -1]).all().item()
    say(f"  {len(rows)} sampled rows exact; properties hold on all {N} rows")
