"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
the CPU oracle on the same seeded inputs, and compare them.

Acceptance (selection ids / attention output), from the method's contract:
  * pooled vectors: bit-exact (both sides round the float64 mean once);
  * selected block ids: bit-exact, except where the oracle's boundary scores
    (the k-th and (k+1)-th of a top-k) tie within 1e-5 relative;
  * attention output given the same mask: max-abs <= 2e-2, mean-abs <= 2e-3,
    and relative L2 <= 1e-2; lse within 2e-3 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf
from oracle import lf_oracle as O

TIE_REL = 1e-5
MAX_ABS, MEAN_ABS, REL_L2 = 2e-2, 2e-3, 1e-2
# lse: the kernel sums its float32 probabilities (float32 accumulation of
# exp2 values), so its log normaliser is within float32 rounding of the
# oracle's; 2e-3 absolute leaves room for the bf16 inputs' score rounding.
LSE_ABS = 2e-3


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def device_inputs(w: I.Workload, x: dict):
    return to_dev(x["q"], w.dtype), to_dev(x["k_cache"], w.dtype), to_dev(x["v_cache"], w.dtype)


def gpu_compress_select(w: I.Workload, x: dict, k_frames: int, k_blocks: int, dev=None):
    g = lf.geom_of(w)
    q, kc, vc = dev if dev is not None else device_inputs(w, x)
    bufs = lf.Buffers(g, k_frames, k_blocks, with_lse=True)
    lf.lf_compress(g, q, kc, x["frame_slot"], bufs.q_blk, bufs.k_blk, bufs.k_frm)
    lf.lf_select(g, bufs.q_blk, bufs.k_blk, bufs.k_frm, k_frames, k_blocks, bufs.sel_frames, bufs.sel_blocks,
                 bufs.n_sel)
    torch.cuda.synchronize()
    return g, (q, kc, vc), bufs


def gpu_attention(w, g, dev, x, sel_blocks: np.ndarray, n_sel: np.ndarray, scale: float):
    q, kc, vc = dev
    sb = torch.from_numpy(np.ascontiguousarray(sel_blocks, np.int32)).cuda()
    ns = torch.from_numpy(np.ascontiguousarray(n_sel, np.int32)).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_compress_select(w: I.Workload, x: dict, k_frames: int, k_blocks: int):
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames,
                   w.hist_frames)
    s = O.select(c["q_blk"], c["k_blk"], c["k_frm"], w.hist_frames, w.n_sink, w.blocks_per_frame, k_frames,
                 k_blocks)
    return c, s


def assert_pooled_bit_exact(bufs, c):
    for name in ("q_blk", "k_blk", "k_frm"):
        got = getattr(bufs, name).cpu().numpy()
        want = c[name]
        assert got.shape == want.shape, name
        bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, f"{name}: {len(bad)} values differ, first at {bad[0].tolist()}: " \
                              f"{got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}"


def _boundary_tie(scores: np.ndarray, k: int) -> bool:
    s = np.sort(np.asarray(scores, np.float64))[::-1]
    if k <= 0 or k >= len(s):
        return False
    a, b = s[k - 1], s[k]
    return abs(a - b) <= TIE_REL * max(abs(a), abs(b))


def compare_selection(w: I.Workload, bufs, s: dict, k_frames: int, k_blocks: int):
    """Returns (n_checked, n_excused, list of unexcused mismatches)."""
    kf, kb = O.effective_k(w.hist_frames, w.n_sink, w.blocks_per_frame, k_frames, k_blocks)
    g_sel = bufs.sel_blocks.cpu().numpy()
    g_n = bufs.n_sel.cpu().numpy()
    g_fr = bufs.sel_frames.cpu().numpy()
    r_sel, r_n, r_fr = s["sel_blocks"], s["n_sel"], s["sel_frames"]
    B, H, nqb = r_n.shape
    excused, bad = 0, []
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                n = r_n[b, h, qb]
                same = g_n[b, h, qb] == n and np.array_equal(g_sel[b, h, qb, :n], r_sel[b, h, qb, :n])
                same = same and np.all(g_sel[b, h, qb, n:] == -1)
                if same and kf > 0:
                    same = np.array_equal(g_fr[b, h, qb, :kf], r_fr[b, h, qb, :kf])
                if same:
                    continue
                if _boundary_tie(s["frame_scores"][b, h, qb], kf):
                    excused += 1
                    continue
                tie_b = any(_boundary_tie(s["block_scores"][b, h, qb, f], kb) for f in r_fr[b, h, qb, :kf])
                if tie_b and np.array_equal(g_fr[b, h, qb, :kf], r_fr[b, h, qb, :kf]):
                    excused += 1
                    continue
                bad.append((b, h, qb, g_sel[b, h, qb, :g_n[b, h, qb]].tolist(), r_sel[b, h, qb, :n].tolist()))
    return B * H * nqb, excused, bad


def sample_qblocks(w: I.Workload, n_random: int = 4, seed: int = 0):
    rng = np.random.default_rng(seed)
    nb, nqb = w.blocks_per_frame, w.n_qblocks
    picks = {0, nb - 1, min(nb, nqb - 1), nqb - 1}
    picks |= set(rng.integers(0, nqb, n_random).tolist())
    heads = sorted({0, w.heads - 1, int(rng.integers(0, w.heads))})
    batches = sorted({0, w.batch - 1})
    return [(b, h, qb) for b in batches for h in heads for qb in sorted(picks)]


def sample_every_head(w: I.Workload, per_head: int = 2, seed: int = 0):
    """Query blocks covering every (batch, head): per head `per_head` spread query blocks (a different
    residue of the head's query blocks each time), and the first and the last three query blocks of every
    head, where ragged frames and work-list tails sit."""
    rng = np.random.default_rng(seed)
    nqb = w.n_qblocks
    out = []
    for b in range(w.batch):
        for h in range(w.heads):
            picks = {0, max(nqb - 3, 0), max(nqb - 2, 0), nqb - 1}
            picks |= set(int(v) for v in rng.integers(0, nqb, per_head))
            picks.add((h * 7 + b) % nqb)
            out += [(b, h, qb) for qb in sorted(picks)]
    return out


def qblock_rows(w: I.Workload, qb: int):
    fc, j = divmod(qb, w.blocks_per_frame)
    s = fc * w.tokens_per_frame + j * w.block
    e = fc * w.tokens_per_frame + min((j + 1) * w.block, w.tokens_per_frame)
    return slice(s, e)


def compare_attention(w: I.Workload, x: dict, out: np.ndarray, lse: np.ndarray, sel_blocks, n_sel, scale: float,
                      qblocks):
    a = O.attention(x["q"], x["k_cache"], x["v_cache"], x["frame_slot"], sel_blocks, n_sel, w.tokens_per_frame,
                    w.block, w.chunk_frames, w.hist_frames, scale, qblocks=qblocks)
    rows_got, rows_ref, lse_err = [], [], 0.0
    for (b, h, qb) in qblocks:
        r = qblock_rows(w, qb)
        rows_got.append(out[b, h, r])
        rows_ref.append(a["out"][b, h, r])
        lse_err = max(lse_err, float(np.max(np.abs(lse[b, h, r] - a["lse"][b, h, r]))))
    got = np.concatenate(rows_got).astype(np.float64)
    ref = np.concatenate(rows_ref)
    err = np.abs(got - ref)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)), "lse_abs": lse_err,
             "rows": int(got.shape[0])}
    assert np.all(np.isfinite(got)), "non-finite output"
    assert stats["max_abs"] <= MAX_ABS and stats["mean_abs"] <= MEAN_ABS, stats
    assert stats["rel_l2"] <= REL_L2, stats
    assert stats["lse_abs"] <= LSE_ABS, stats
    return stats


def gpu_select_blocks(g, bufs, k_total: int):
    """Single-level selection on the GPU from already pooled q_blk / k_blk in bufs."""
    m = max(lf.lf_max_sel_1d(g, k_total), 1)
    sel = torch.empty((g.batch, g.heads, g.n_qblocks, m), dtype=torch.int32, device="cuda")
    n = torch.empty((g.batch, g.heads, g.n_qblocks), dtype=torch.int32, device="cuda")
    lf.lf_select_blocks(g, bufs.q_blk, bufs.k_blk, k_total, sel, n)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), n.cpu().numpy()


def compare_selection_1d(g_sel, g_n, r: dict, k_total: int):
    """Returns (n_checked, n_excused, unexcused mismatches) for the single-level variant."""
    r_sel, r_n, sc = r["sel_blocks"], r["n_sel"], r["scores"]
    k = min(k_total, sc.shape[-1])
    B, H, nqb = r_n.shape
    excused, bad = 0, []
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                n = r_n[b, h, qb]
                same = g_n[b, h, qb] == n and np.array_equal(g_sel[b, h, qb, :n], r_sel[b, h, qb, :n])
                same = same and np.all(g_sel[b, h, qb, n:] == -1)
                if same:
                    continue
                if _boundary_tie(sc[b, h, qb], k):
                    excused += 1
                    continue
                bad.append((b, h, qb, g_sel[b, h, qb, :g_n[b, h, qb]].tolist(), r_sel[b, h, qb, :n].tolist()))
    return B * H * nqb, excused, bad
