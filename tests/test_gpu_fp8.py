"""GPU parity of the FP8 attention variant (lf_block_sparse_attn_fp8).

Queries and keys are quantised on the host to MX-FP8 (E4M3 codes, one E8M0
scale per 32 channels; inputs.mx_quantize). The oracle computes the same
block-sparse attention in float64 on exactly the values those codes and
scales stand for (oracle.attention_fp8), with the oracle's own selection, so
the masks are shared. FP8 products are exact in float32, so the kernel's
score error is only its float32 accumulation; the softmax, P (bf16) and the
bf16 V product are the bf16 kernel's. The bar is therefore the bf16 bar of
tests/parity.py (max-abs 2e-2, mean-abs 2e-3, rel-L2 1e-2, lse 4e-3).

The quantisation error itself (FP8 attention against the bf16 inputs'
attention) is printed for information; it is a property of the format, not
of the kernel.
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf
from oracle import lf_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _quantised(x):
    q8, qs = I.mx_quantize(x["q"])
    k8, ks = I.mx_quantize(x["k_cache"])
    return q8, qs, k8, ks


def _run(w, qblocks=None, scale_mult=1.0, seed=None):
    _say(f"[fp8] {w.name} B={w.batch} H={w.heads} T={w.tokens_per_frame} b={w.block} Fc={w.chunk_frames} "
         f"Fh={w.hist_frames} scale_mult={scale_mult}")
    x = I.make_inputs(w, seed=seed)
    g = lf.geom_of(w)
    q8, qs, k8, ks = _quantised(x)
    _, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    scale = scale_mult / math.sqrt(w.head_dim)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in
           (("q8", q8), ("qs", qs), ("k8", k8), ("ks", ks))}
    vc = P.to_dev(x["v_cache"], "bf16")
    sb = torch.from_numpy(np.ascontiguousarray(s["sel_blocks"], np.int32)).cuda()
    ns = torch.from_numpy(np.ascontiguousarray(s["n_sel"], np.int32)).cuda()
    out = torch.empty((w.batch, w.heads, w.q_len, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.heads, w.q_len), dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn_fp8(g, dev["q8"], dev["qs"], dev["k8"], dev["ks"], vc, x["frame_slot"], sb, ns, scale,
                                out, lse)
    torch.cuda.synchronize()
    got, got_lse = out.float().cpu().numpy(), lse.cpu().numpy()
    if qblocks is None:
        qblocks = [(b, h, qb) for b in range(w.batch) for h in range(w.heads) for qb in range(w.n_qblocks)]
    a = O.attention_fp8(q8, qs, k8, ks, x["v_cache"], x["frame_slot"], s["sel_blocks"], s["n_sel"],
                        w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames, scale, qblocks=qblocks)
    ref_bf16 = O.attention(x["q"], x["k_cache"], x["v_cache"], x["frame_slot"], s["sel_blocks"], s["n_sel"],
                           w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames, scale, qblocks=qblocks)
    rows_got, rows_ref, rows_bf, lse_err = [], [], [], 0.0
    for (b, h, qb) in qblocks:
        r = P.qblock_rows(w, qb)
        rows_got.append(got[b, h, r])
        rows_ref.append(a["out"][b, h, r])
        rows_bf.append(ref_bf16["out"][b, h, r])
        lse_err = max(lse_err, float(np.max(np.abs(got_lse[b, h, r] - a["lse"][b, h, r]))))
    gv = np.concatenate(rows_got).astype(np.float64)
    rv = np.concatenate(rows_ref)
    bv = np.concatenate(rows_bf)
    err = np.abs(gv - rv)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "rel_l2": float(np.linalg.norm(gv - rv) / max(np.linalg.norm(rv), 1e-300)), "lse_abs": lse_err,
             "rows": int(gv.shape[0]),
             "quant_rel_l2": float(np.linalg.norm(rv - bv) / max(np.linalg.norm(bv), 1e-300))}
    _say(f"[fp8] {stats}")
    assert np.all(np.isfinite(gv)), "non-finite output"
    assert stats["max_abs"] <= P.MAX_ABS and stats["mean_abs"] <= P.MEAN_ABS, stats
    assert stats["rel_l2"] <= P.REL_L2 and stats["lse_abs"] <= P.LSE_ABS, stats
    return stats


def _odd(T, b, Fc=2, Fh=4, H=2, kf=2, kb=2, n_sink=1, slots=None, dist="normal"):
    return I.Workload(name=f"fp8_{T}_{b}_{Fh}", batch=1, heads=H, head_dim=128, grid=(1, T), block=b,
                      chunk_frames=Fc, hist_frames=Fh, n_sink=n_sink if Fh > 0 else 0,
                      cache_slots=slots if slots is not None else Fh + Fc + 2, dtype="bf16", k_frames=kf,
                      k_blocks=kb, sparsity=float("nan"), seed=9, dist=dist, chunk_index=4)


@pytest.mark.parametrize("T,b", [(200, 64), (130, 64), (100, 48), (77, 40), (64, 64), (33, 33), (77, 16), (100, 32),
                                 (200, 96), (300, 128), (128, 128), (130, 65)])
def test_fp8_odd_geometries(T, b):
    """Ragged last blocks, blocks shorter than a 64-key tile, one-block frames; blocks of up to 32 keys (four
    query blocks per workgroup) and of 65-128 keys (two 64-key tiles per block) take the double-buffered walk."""
    _run(_odd(T, b))


def test_fp8_empty_history():
    _run(_odd(150, 64, Fh=0))


def test_fp8_two_batches_many_heads():
    w = _odd(160, 64, H=5).replace(batch=2, name="fp8_b2_h5")
    _run(w)


def test_fp8_sharp_logits():
    """Scores 8x sharper than 1/sqrt(d): the exact (rescaling) path of both halves runs."""
    _run(_odd(200, 64), scale_mult=8.0)


def test_fp8_wan480p_chunk_every_row():
    """The 480p chunk at full size (12 heads, 4680 queries, 6 history frames), every query block."""
    _run(I.WAN480P_CHUNK)


def test_fp8_wide_head_every_head():
    """40 heads, 3600-token frames, 128-token blocks: the first and last three and spread query blocks of
    every head."""
    w = I.WIDE_HEAD
    _run(w, qblocks=P.sample_every_head(w, per_head=1))


def test_fp8_long_history_sink_every_head():
    w = I.LONG_HISTORY_SINK
    _run(w, qblocks=P.sample_every_head(w, per_head=1))


def test_fp8_selection_lists_near_lf_max_sel():
    """508 selected history blocks per query block (254 frames, 2 of 4 blocks each)."""
    w = _odd(256, 64, Fc=1, Fh=254, H=1, kf=254, kb=2, n_sink=0, slots=255).replace(chunk_index=300)
    _run(w)


def _fp8_call(w, x, q8, qs, k8, ks, sel, nsel, scale):
    g = lf.geom_of(w)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q8, qs, k8, ks)]
    vc = P.to_dev(x["v_cache"], "bf16")
    sb = torch.from_numpy(np.ascontiguousarray(sel, np.int32)).cuda()
    ns = torch.from_numpy(np.ascontiguousarray(nsel, np.int32)).cuda()
    out = torch.empty((w.batch, w.heads, w.q_len, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lf.lf_block_sparse_attn_fp8(g, *dev, vc, x["frame_slot"], sb, ns, scale, out, None)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("T,b", [(100, 16), (200, 64), (300, 128)])
def test_fp8_ignored_ids_and_unsorted_lists(T, b):
    """Ids of -1 or out of range and entries past n_sel change nothing (bit for bit); lists in descending
    order (no shared tiles in the union walk of b = 16) still match the oracle."""
    w = _odd(T, b, Fh=5, kf=3, kb=2)
    _say(f"[fp8] ignored/unsorted {w.name}")
    x = I.make_inputs(w)
    q8, qs, k8, ks = _quantised(x)
    _, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    scale = 1.0 / math.sqrt(w.head_dim)
    base = _fp8_call(w, x, q8, qs, k8, ks, s["sel_blocks"], s["n_sel"], scale)
    m = s["sel_blocks"].shape[-1]
    noisy = np.full(s["sel_blocks"].shape[:-1] + (m + 6,), 10 ** 6, np.int32)
    noisy[..., 1:m + 1] = s["sel_blocks"]
    noisy[..., 0] = -1
    noisy[..., m + 1] = w.hist_frames * w.blocks_per_frame
    got = _fp8_call(w, x, q8, qs, k8, ks, noisy, s["n_sel"] + 2, scale)
    assert np.array_equal(got, base)
    rev = s["sel_blocks"].copy()
    for idx in np.ndindex(rev.shape[:-1]):
        n = s["n_sel"][idx]
        rev[idx][:n] = rev[idx][:n][::-1].copy()
    got_rev = _fp8_call(w, x, q8, qs, k8, ks, rev, s["n_sel"], scale)
    qbs = [(0, h, qb) for h in range(w.heads) for qb in range(w.n_qblocks)]
    a = O.attention_fp8(q8, qs, k8, ks, x["v_cache"], x["frame_slot"], s["sel_blocks"], s["n_sel"],
                        w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames, scale, qblocks=qbs)
    err = np.abs(got_rev.astype(np.float64) - a["out"])
    assert err.max() <= P.MAX_ABS and err.mean() <= P.MEAN_ABS, (err.max(), err.mean())
    rel = float(np.linalg.norm(got_rev - a["out"]) / np.linalg.norm(a["out"]))
    assert rel <= P.REL_L2, rel
