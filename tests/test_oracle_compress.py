"""Pins of the oracle's token compression (mean pooling per block and per frame).

Pinned against closed forms (means of arithmetic progressions), exact rational
arithmetic, and the block/frame consistency invariant. Light Forcing technical
summary 2.2 ("token compression": mean pooling at block and frame granularity).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import lf_oracle as O


@pytest.mark.parametrize("T,b,n,last", [(1560, 64, 25, (1536, 1560)), (3600, 128, 29, (3584, 3600)),
                                        (64, 16, 4, (48, 64)), (100, 100, 1, (0, 100)), (5, 8, 1, (0, 5))])
def test_block_ranges_ceil_partition(T, b, n, last):
    r = O.block_ranges(T, b)
    assert len(r) == n and r[-1] == last and r[0][0] == 0
    assert all(r[i][1] == r[i + 1][0] for i in range(n - 1))  # contiguous, no straddling
    assert sum(e - s for s, e in r) == T


def _progression_inputs(B, H, T, d, F_c, S):
    t = np.arange(F_c * T, dtype=np.float32)[:, None]
    dd = np.arange(d, dtype=np.float32)[None, :]
    q = np.broadcast_to(t + 0.25 * dd, (B, H, F_c * T, d)).copy()
    slot_ids = np.arange(S, dtype=np.float32)[:, None, None]
    tok = np.arange(T, dtype=np.float32)[None, :, None]
    k = np.broadcast_to(1000.0 * slot_ids + tok - 0.5 * dd[None], (B, H, S, T, d)).copy()
    return q, k


@pytest.mark.parametrize("T,b,F_c,F_h", [(60, 16, 2, 3), (64, 16, 1, 4), (1560, 64, 1, 2)])
def test_pool_arithmetic_progression_closed_form(T, b, F_c, F_h):
    """Mean of tokens t = s..e-1 of a progression is (s + e - 1) / 2: pins ranges, ragged tails,
    the slot indirection and the divisor (valid-token count)."""
    B, H, d = 1, 2, 8
    S = F_h + F_c + 1
    q, k = _progression_inputs(B, H, T, d, F_c, S)
    slots = np.random.default_rng(T).permutation(S)[:F_h + F_c].astype(np.int32)
    assert len(set(slots.tolist())) == len(slots)
    c = O.compress(q, k, slots, T, b, F_c, F_h)
    ranges = O.block_ranges(T, b)
    nb = len(ranges)
    dd = np.arange(d) * 0.25
    for fc in range(F_c):
        for j, (s, e) in enumerate(ranges):
            want = (fc * T + s + fc * T + e - 1) / 2.0 + dd
            np.testing.assert_array_equal(c["q_blk"][0, 1, fc * nb + j], want.astype(np.float32))
    for f in range(F_h):
        for j, (s, e) in enumerate(ranges):
            want = 1000.0 * slots[f] + (s + e - 1) / 2.0 - 2 * dd
            np.testing.assert_array_equal(c["k_blk"][0, 0, f * nb + j], want.astype(np.float32))
        np.testing.assert_array_equal(c["k_frm"][0, 1, f], (1000.0 * slots[f] + (T - 1) / 2.0 - 2 * dd).astype(np.float32))


def test_pool_is_exact_mean_rounded_once():
    """Against exact rational means: the pooled value is the float32 nearest the exact mean
    (to within the one float64 rounding before it)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((37, 5)) * np.exp2(rng.integers(-12, 12, (37, 5)))).astype(np.float32)
    got = O.mean_pool(x)
    for dcol in range(5):
        exact = sum(Fraction(float(v)) for v in x[:, dcol]) / 37
        nearest = np.float32(float(exact))
        # float32 nearest to the exact mean, or (double rounding) its neighbour
        assert got[dcol] in (nearest, np.nextafter(nearest, np.float32(np.inf)),
                             np.nextafter(nearest, np.float32(-np.inf)))
        assert abs(float(got[dcol]) - float(exact)) <= float(np.spacing(np.float32(abs(float(exact)))))


def test_frame_mean_is_token_weighted_block_mean():
    rng = np.random.default_rng(3)
    T, b, d = 1560, 64, 16
    k = rng.standard_normal((1, 1, 3, T, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    c = O.compress(q, k, [2, 0, 1], T, b, 1, 2)
    ranges = O.block_ranges(T, b)
    nb = len(ranges)
    for f in range(2):
        w = np.array([e - s for s, e in ranges], np.float64)
        recon = (w[:, None] * c["k_blk"][0, 0, f * nb:(f + 1) * nb].astype(np.float64)).sum(0) / T
        np.testing.assert_allclose(c["k_frm"][0, 0, f], recon, rtol=0, atol=1e-6)
        # and it really is frame f's slot, not another frame
        np.testing.assert_allclose(c["k_frm"][0, 0, f], k[0, 0, [2, 0][f]].astype(np.float64).mean(0), atol=1e-6)


def test_constant_tokens_pool_to_the_constant():
    q = np.full((1, 1, 48, 4), 0.3, np.float32)
    k = np.full((1, 1, 2, 24, 4), -1.75, np.float32)
    c = O.compress(q[:, :, :24], k, [1, 0], 24, 10, 1, 1)
    assert np.all(c["q_blk"] == np.float32(0.3)) and np.all(c["k_blk"] == np.float32(-1.75))
