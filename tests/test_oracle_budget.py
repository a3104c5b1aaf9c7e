"""Pins of the oracle's chunk-aware growth (CAG) budget.

Light Forcing technical summary 2.1: s_i = s_base - alpha_i * beta with
alpha_i ~ 1/sqrt(noise level), beta tuned to the target; press summary
section 2: earlier (lower-noise) chunks get lower sparsity, and CAG is
compared against uniform allocation under the same total budget; section 1:
seven chunks with the first one dense.
beta is pinned by solving the mean constraint numerically (scipy brentq),
not by the closed form the oracle uses.
"""
import math

import numpy as np
import pytest
from scipy.optimize import brentq

from block_sparse_attention_lf_amd import inputs as I
from oracle import lf_oracle as O

R = I.CHUNK_ROLLOUT


def _rollout(weight=None, s_target=0.8):
    sig = R.sigmas()
    n = R.n_chunks
    return O.chunk_budget(sig, weight or [1.0] * n, [True] + [False] * (n - 1), R.s_base, s_target,
                          [R.chunk_frames * i for i in range(n)], [0] * n, R.blocks_per_frame, R.k_frames_min)


def test_beta_solves_the_mean_constraint_numerically():
    sig = R.sigmas()[1:]
    f = lambda beta: np.mean([R.s_base - beta / math.sqrt(s) for s in sig]) - 0.8
    beta_num = brentq(f, -10, 10, xtol=1e-15)
    out = _rollout()
    assert abs(out["beta"] - beta_num) < 1e-12
    assert abs(np.mean(out["sparsity"][1:]) - 0.8) < 1e-12
    assert out["sparsity"][0] == 0.0


def test_weighted_reading_meets_weighted_mean():
    w = [float(i) for i in range(R.n_chunks)]  # e.g. history-proportional weights
    out = _rollout(weight=w)
    s = out["sparsity"]
    assert abs(sum(w[i] * s[i] for i in range(1, 7)) / sum(w[1:]) - 0.8) < 1e-12


def test_sparsity_grows_with_noise_level():
    s = _rollout()["sparsity"][1:]
    assert all(a < b for a, b in zip(s, s[1:]))
    assert _rollout()["beta"] > 0


def test_target_equal_to_base_is_uniform_allocation():
    out = _rollout(s_target=R.s_base)
    assert out["beta"] == 0.0
    assert all(abs(x - R.s_base) < 1e-15 for x in out["sparsity"][1:])


def test_topk_sizes_spend_the_budget():
    out = _rollout()
    nb = R.blocks_per_frame
    for i in range(1, R.n_chunks):
        F = R.chunk_frames * i
        budget = (1 - out["sparsity"][i]) * F * nb
        kf, kb = out["k_frames"][i], out["k_blocks"][i]
        assert R.k_frames_min <= kf <= F and 1 <= kb <= nb
        assert abs(kf * kb - budget) <= kf / 2 + 1e-9  # rounding of k_b only
        assert kf == max(R.k_frames_min, math.ceil(budget / nb - 1e-9))
    assert out["k_frames"][0] == 0 and out["k_blocks"][0] == 0  # dense first chunk has no history


def test_single_chunk_sizing_matches_workload_tables():
    """The sizing rule reproduces the fixed k of the single-call workloads from their sparsity."""
    for w in (I.WAN480P_CHUNK, I.LONG_HISTORY_SINK, I.WIDE_HEAD, I.TINY_FP32):
        out = O.chunk_budget([1.0], [1.0], [False], w.sparsity, w.sparsity, [w.hist_frames], [w.n_sink],
                             w.blocks_per_frame, w.k_frames)
        assert (out["k_frames"][0], out["k_blocks"][0]) == (w.k_frames, w.k_blocks), w.name


def test_dense_chunk_with_history_takes_everything():
    out = O.chunk_budget([0.5, 1.0], [1, 1], [True, False], 0.9, 0.8, [4, 4], [1, 1], 5, 1)
    assert out["k_frames"][0] == 3 and out["k_blocks"][0] == 5 and out["sparsity"][0] == 0.0
