"""Pins of the oracle's two-stage mask selection.

Light Forcing technical summary 2.2 ("two-stage mask selection"): per query
block, frames are ranked by inner product with frame-level keys, then blocks
inside each chosen frame by block-level keys; selection cost does not depend
on the history length. Pinned by brute-force subset enumeration, planted
frames, duplicate frames (lowest index wins), and invariants.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import lf_oracle as O


def brute_top_k(scores, k):
    """Max-sum k-subset; among equal sums the lexicographically smallest index tuple."""
    best = None
    for sub in itertools.combinations(range(len(scores)), k):
        s = math.fsum(scores[i] for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    return list(best[1]) if best else []


@pytest.mark.parametrize("seed", range(40))
def test_top_k_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    k = int(rng.integers(0, n + 1))
    scores = rng.integers(-3, 4, n).astype(np.float64)  # many exact ties
    assert sorted(O.top_k_desc(scores, k).tolist()) == brute_top_k(scores.tolist(), k)


def _dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n_sink", [0, 1])
def test_select_matches_brute_force(seed, n_sink):
    rng = np.random.default_rng(100 + seed)
    B, H, nqb, d, F, nb, kf, kb = 1, 2, 3, 8, 5, 4, 2, 2
    q_blk = rng.standard_normal((B, H, nqb, d)).astype(np.float32)
    k_blk = rng.standard_normal((B, H, F * nb, d)).astype(np.float32)
    k_frm = rng.standard_normal((B, H, F, d)).astype(np.float32)
    r = O.select(q_blk, k_blk, k_frm, F, n_sink, nb, kf, kb)
    for h in range(H):
        for qb in range(nqb):
            qv = q_blk[0, h, qb]
            cands = list(range(n_sink, F))
            fs = [_dot(qv, k_frm[0, h, f]) for f in cands]
            chosen = [cands[i] for i in brute_top_k(fs, kf)]
            want = [f * nb + j for f in range(n_sink) for j in range(nb)]
            for f in chosen:
                bs = [_dot(qv, k_blk[0, h, f * nb + j]) for j in range(nb)]
                want += [f * nb + j for j in brute_top_k(bs, kb)]
            want = sorted(want)
            n = r["n_sel"][0, h, qb]
            assert n == len(want) == n_sink * nb + kf * kb
            assert r["sel_blocks"][0, h, qb, :n].tolist() == want
            assert r["sel_frames"][0, h, qb].tolist() == sorted(chosen)


def test_planted_frames_are_recovered():
    """Orthogonal plants: frame f carries u_f strongly; a query block built from u_2 + u_4 picks 2 and 4."""
    d, F, nb = 16, 6, 3
    basis = np.eye(d, dtype=np.float32)
    k_frm = np.stack([basis[f] * 0.1 for f in range(F)])
    k_frm[2] = basis[2] * 5
    k_frm[4] = basis[4] * 3
    k_blk = np.zeros((F * nb, d), np.float32)
    for f in range(F):
        k_blk[f * nb + (f % nb)] = basis[f] * 2  # one hot block per frame
    q = (basis[2] + basis[4])[None]
    r = O.select(q[None, None], k_blk[None, None], k_frm[None, None], F, 0, nb, 2, 1)
    assert r["sel_frames"][0, 0, 0].tolist() == [2, 4]
    assert r["sel_blocks"][0, 0, 0, :2].tolist() == [2 * nb + 2, 4 * nb + 1]


def test_duplicate_frames_lowest_index_wins():
    d, F, nb = 8, 5, 2
    rng = np.random.default_rng(5)
    k_frm = rng.standard_normal((F, d)).astype(np.float32) * 0.01
    k_frm[1] = k_frm[3] = np.ones(d, np.float32)
    k_blk = np.zeros((F * nb, d), np.float32)  # all block scores tie at 0
    q = np.ones((1, 1, 1, d), np.float32)
    r = O.select(q, k_blk[None, None], k_frm[None, None], F, 0, nb, 1, 1)
    assert r["sel_frames"][0, 0, 0].tolist() == [1]
    assert r["sel_blocks"][0, 0, 0, :1].tolist() == [1 * nb + 0]  # tied blocks: lowest j


def test_sink_frames_forced_and_not_candidates():
    rng = np.random.default_rng(9)
    d, F, nb = 8, 6, 3
    q = rng.standard_normal((1, 1, 2, d)).astype(np.float32)
    k_frm = rng.standard_normal((1, 1, F, d)).astype(np.float32)
    k_frm[0, 0, 0] = q[0, 0, 0] * 100  # the sink would win any ranking
    k_blk = rng.standard_normal((1, 1, F * nb, d)).astype(np.float32)
    r = O.select(q, k_blk, k_frm, F, 1, nb, 2, 1)
    for qb in range(2):
        ids = r["sel_blocks"][0, 0, qb, :r["n_sel"][0, 0, qb]].tolist()
        assert ids[:nb] == list(range(nb))
        assert 0 not in r["sel_frames"][0, 0, qb].tolist()
        assert len(ids) == nb + 2


@pytest.mark.parametrize("F", [3, 6, 12, 21])
def test_selected_count_does_not_grow_with_history(F):
    rng = np.random.default_rng(F)
    d, nb = 8, 5
    q = rng.standard_normal((1, 1, 4, d)).astype(np.float32)
    r = O.select(q, rng.standard_normal((1, 1, F * nb, d)).astype(np.float32),
                 rng.standard_normal((1, 1, F, d)).astype(np.float32), F, 1, nb, 2, 3)
    assert np.all(r["n_sel"] == nb + 2 * 3)


def test_k_clamped_to_what_exists():
    rng = np.random.default_rng(1)
    d, F, nb = 4, 3, 2
    r = O.select(rng.standard_normal((1, 1, 1, d)).astype(np.float32),
                 rng.standard_normal((1, 1, F * nb, d)).astype(np.float32),
                 rng.standard_normal((1, 1, F, d)).astype(np.float32), F, 1, nb, 5, 7)
    assert r["n_sel"][0, 0, 0] == F * nb  # everything: sink + both candidates in full


def test_empty_history_selects_nothing():
    r = O.select(np.ones((1, 1, 2, 4), np.float32), np.zeros((1, 1, 0, 4), np.float32),
                 np.zeros((1, 1, 0, 4), np.float32), 0, 0, 3, 3, 2)
    assert np.all(r["n_sel"] == 0)


def test_invariant_to_common_key_shift_and_power_of_two_query_scale():
    rng = np.random.default_rng(11)
    d, F, nb, nqb = 16, 7, 5, 4
    q = rng.standard_normal((1, 2, nqb, d)).astype(np.float32)
    kb = rng.standard_normal((1, 2, F * nb, d)).astype(np.float32)
    kf = rng.standard_normal((1, 2, F, d)).astype(np.float32)
    base = O.select(q, kb, kf, F, 0, nb, 3, 2)
    scaled = O.select(q * np.float32(8.0), kb, kf, F, 0, nb, 3, 2)
    assert np.array_equal(base["sel_blocks"], scaled["sel_blocks"])
    # A shift c of every key moves all of one query block's scores by <q, c>; use a
    # dyadic shift so that the shifted scores stay exact.
    c = np.float32(0.5) * np.sign(rng.standard_normal(d)).astype(np.float32)
    shifted = O.select(q, kb + c, kf + c, F, 0, nb, 3, 2)
    assert np.array_equal(base["sel_blocks"], shifted["sel_blocks"])


# ---------------------------------------------------------------------------
# Single-level ("1D") selection, the ablation baseline (press summary,
# section 4): one top-k over all non-sink history blocks.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_select_blocks_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Fh, nb, d = 4, 3, 4
    ns = int(seed % 2)
    q_blk = rng.integers(-2, 3, size=(1, 1, 2, d)).astype(np.float32)
    k_blk = rng.integers(-2, 3, size=(1, 1, Fh * nb, d)).astype(np.float32)  # integer grid: many exact ties
    ncand = (Fh - ns) * nb
    for k in range(ncand + 2):
        r = O.select_blocks(q_blk, k_blk, Fh, ns, nb, k)
        for qb in range(2):
            sc = [float(np.dot(q_blk[0, 0, qb].astype(np.float64), k_blk[0, 0, i].astype(np.float64)))
                  for i in range(ns * nb, Fh * nb)]
            want = list(range(ns * nb)) + sorted(ns * nb + i for i in brute_top_k(sc, min(k, ncand)))
            n = int(r["n_sel"][0, 0, qb])
            assert r["sel_blocks"][0, 0, qb, :n].tolist() == want


def test_select_blocks_follows_a_plant_the_frame_stage_cannot():
    """All four best blocks sit in one frame: the single-level top-4 takes them
    all, while the two-stage selection with the same budget (2 frames x 2
    blocks) can take only two of them."""
    Fh, nb, d = 4, 4, 8
    rng = np.random.default_rng(7)
    q_blk = np.zeros((1, 1, 1, d), np.float32)
    q_blk[..., 0] = 1.0
    k_blk = rng.normal(0, 0.1, size=(1, 1, Fh * nb, d)).astype(np.float32)
    k_blk[0, 0, 2 * nb:3 * nb, 0] += 5.0          # frame 2's blocks dominate
    k_frm = k_blk.reshape(1, 1, Fh, nb, d).mean(axis=3).astype(np.float32)
    one = O.select_blocks(q_blk, k_blk, Fh, 0, nb, 4)
    assert one["sel_blocks"][0, 0, 0].tolist() == list(range(2 * nb, 3 * nb))
    two = O.select(q_blk, k_blk, k_frm, Fh, 0, nb, 2, 2)
    got = set(two["sel_blocks"][0, 0, 0, :int(two["n_sel"][0, 0, 0])].tolist())
    assert len(got & set(range(2 * nb, 3 * nb))) == 2 and len(got) == 4


def test_select_blocks_all_blocks_and_sinks():
    rng = np.random.default_rng(3)
    Fh, nb, d, ns = 5, 4, 8, 2
    q_blk = rng.normal(size=(1, 2, 3, d)).astype(np.float32)
    k_blk = rng.normal(size=(1, 2, Fh * nb, d)).astype(np.float32)
    r = O.select_blocks(q_blk, k_blk, Fh, ns, nb, 10 ** 6)
    assert (r["n_sel"] == Fh * nb).all()
    assert (r["sel_blocks"] == np.arange(Fh * nb)).all()
    assert O.max_selected_1d(Fh, ns, nb, 5) == ns * nb + 5
    r0 = O.select_blocks(q_blk, k_blk, Fh, ns, nb, 0)
    assert (r0["n_sel"] == ns * nb).all()


def test_select_blocks_invariant_to_common_key_shift():
    rng = np.random.default_rng(11)
    Fh, nb, d = 6, 5, 16
    q_blk = rng.normal(size=(1, 1, 4, d)).astype(np.float32)
    k_blk = rng.normal(size=(1, 1, Fh * nb, d)).astype(np.float32)
    shift = rng.normal(size=(d,)).astype(np.float32)
    a = O.select_blocks(q_blk, k_blk, Fh, 1, nb, 7)
    b = O.select_blocks(q_blk, (k_blk + shift).astype(np.float32), Fh, 1, nb, 7)
    # scores move by <q, shift> for every candidate alike: same selection unless
    # float32 rounding of the shifted keys reorders a near-tie
    gaps = np.diff(np.sort(a["scores"], axis=-1), axis=-1)
    if np.min(gaps) > 1e-3:
        assert np.array_equal(a["sel_blocks"], b["sel_blocks"])
