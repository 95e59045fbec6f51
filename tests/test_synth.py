"""The seeded input generator: determinism, bf16 rounding, id structure."""
import math

import numpy as np
import pytest

from synth import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_inputs,
                   make_teacher_cache)


def test_bf16_rne_known_patterns():
    # exact values survive; halfway cases go to even; overflow rounds to inf
    x = np.array([1.0, -2.5, 0.0, -0.0, 3.140625], dtype=np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)), x)
    one = np.float32(1.0).view(np.uint32)
    halfway_down = np.array([one + 0x8000], dtype=np.uint32).view(np.float32)  # 1 + 2^-8: tie, even is 1.0
    halfway_up = np.array([one + 0x18000], dtype=np.uint32).view(np.float32)   # tie, rounds up to even
    above = np.array([one + 0x8001], dtype=np.uint32).view(np.float32)
    assert f32_to_bf16_bits(halfway_down)[0] == 0x3F80
    assert f32_to_bf16_bits(halfway_up)[0] == 0x3F82
    assert f32_to_bf16_bits(above)[0] == 0x3F81
    big = np.array([3.4e38], dtype=np.float32)
    assert f32_to_bf16_bits(big)[0] == 0x7F80


def test_bf16_rne_edge_bit_patterns():
    # largest finite values, infinities, the top of the bit range (where a 32-bit
    # sum of the rounding bias would wrap) and NaNs: compared with the rounding
    # written out in 64-bit integers
    pats = np.concatenate([
        np.arange(0x7F7F0000, 0x7F810000, 0x1001, dtype=np.uint64),
        np.arange(0xFF7F0000, 0xFF810000, 0x1001, dtype=np.uint64),
        np.arange(0xFFFF0000, 0x100000000, 0x111, dtype=np.uint64),
        np.arange(0x7FFF0000, 0x80010000, 0x777, dtype=np.uint64),
        np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFFFFFFF], dtype=np.uint64),
    ]).astype(np.uint32)
    x = pats.view(np.float32)
    u = pats.astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    ref[np.isnan(x)] = 0x7FC0
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_bf16_rne_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_deterministic_and_seed_sensitive():
    cfg = get_config("tiny")
    a = make_inputs(cfg, seed=0)
    b = make_inputs(cfg, seed=0)
    c = make_inputs(cfg, seed=1)
    for k in ("H", "W", "idx", "t"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["H"], c["H"])


def test_tiny_cache_structure():
    cfg = get_config("tiny")
    idx, t = make_teacher_cache(cfg, 0)
    assert idx.shape == (cfg.N, cfg.K) and idx.dtype == np.int32
    assert t.shape == (cfg.N, cfg.K) and t.dtype == np.float32
    assert idx.min() >= 0 and idx.max() < cfg.V
    for row in idx:
        assert len(set(row.tolist())) == cfg.K
    assert np.all(np.diff(t, axis=1) <= 0)
    # N(0, variance 3)
    assert abs(t.std() - math.sqrt(3)) < 0.15


def test_zipf_cache_structure():
    cfg = get_config("toy").replace(N=2048)
    idx, t = make_teacher_cache(cfg, 0)
    assert idx.min() >= 0 and idx.max() < cfg.V
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    # Zipf(1.1) head: rank 1 (id 0) appears in nearly every row, ~46% of ids < 256
    assert (idx == 0).any(axis=1).mean() > 0.99
    frac = (idx < 256).mean()
    assert 0.40 < frac < 0.52
    assert np.all(np.diff(t, axis=1) <= 0)


def test_zipf_perm_is_a_relabelling():
    cfg = get_config("toy").replace(N=256)
    a, _ = make_teacher_cache(cfg, 0)
    b, _ = make_teacher_cache(cfg.replace(ids="zipf_perm"), 0)
    # same multiset structure: identical ids map to identical ids
    m = {}
    for x, y in zip(a.ravel().tolist(), b.ravel().tolist()):
        assert m.setdefault(x, y) == y
    assert (b < 256).mean() < 0.05


def test_weight_scale():
    cfg = get_config("tiny")
    inp = make_inputs(cfg, 0)
    W = bf16_bits_to_f32(inp["W"])
    H = bf16_bits_to_f32(inp["H"])
    assert abs(W.std() * math.sqrt(cfg.D) - 1) < 0.02
    assert abs(H.std() - 1) < 0.02


def test_all_configs_declared():
    assert set(CONFIGS) == {"tiny", "toy", "large_vocab", "long", "very_long"}
    assert CONFIGS["large_vocab"].V == 201088 and CONFIGS["large_vocab"].D == 2880
    assert CONFIGS["very_long"].N == 262144
