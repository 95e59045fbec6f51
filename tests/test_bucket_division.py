"""The bucketing kernel finds the row of cache entry e (of a 256-position
tile, K entries per row) as int((float(e) + 0.5) * (1 / K)) in fp32 instead of
an integer division.  Checked here for every K the library accepts and every
entry of a full tile, in the same fp32 arithmetic: 1.0f / K correctly rounded
(HIP's default fp32 division), then an add and a multiply rounded to nearest
even, then truncation."""
import numpy as np


def test_float_reciprocal_row_equals_integer_division():
    for K in range(1, 257):
        e = np.arange(256 * K, dtype=np.int64)
        invK = np.float32(1.0) / np.float32(K)
        rr = ((e.astype(np.float32) + np.float32(0.5)) * invK).astype(np.int64)
        assert (rr == e // K).all(), K
