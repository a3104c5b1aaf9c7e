"""GPU parity of the backward pass (lf_block_sparse_attn_bwd) against the oracle.

The forward runs on the GPU (its out and lse feed the backward, as in
training); the selection is the oracle's, so both sides use the same masks.
dout is seeded N(0,1), rounded to bf16. dq, dk_cache and dv_cache (float32)
are compared with oracle.attention_grad on the same bf16 values. Tolerance,
per tensor: relative L2 error <= 1e-2 and max-abs error <= 2e-2 * max|ref|.
The GPU rounds P and dS to bf16 (relative 2^-9 each) before the MFMAs and
reads out in bf16; these errors are independent across the summed terms, so
the aggregate stays well under 1e-2. Rows of cache slots the frame table
does not name must come back untouched (their sentinel value).
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

REL_L2, MAX_REL = 1e-2, 2e-2
SENTINEL = 12345.0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(name, got, want):
    err = got - want
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-30))
    mx = float(np.max(np.abs(err))) / max(float(np.max(np.abs(want))), 1e-30)
    _say(f"[bwd] {name}: rel_l2 {rel:.2e}, max_abs/max|ref| {mx:.2e}")
    assert np.all(np.isfinite(got)), name
    assert rel <= REL_L2 and mx <= MAX_REL, (name, rel, mx)


def _run(w, heads_checked=None, seed=17, sel_fn=None):
    _say(f"[bwd] {w.name} B={w.batch} H={w.heads} d={w.head_dim} T={w.tokens_per_frame} b={w.block} "
         f"Fc={w.chunk_frames} Fh={w.hist_frames}")
    x = I.make_inputs(w)
    g = lf.geom_of(w)
    dev = P.device_inputs(w, x)
    q, kc, vc = dev
    _, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    if sel_fn is not None:
        s = sel_fn(w, s)
    sb = torch.from_numpy(np.ascontiguousarray(s["sel_blocks"], np.int32)).cuda()
    ns = torch.from_numpy(np.ascontiguousarray(s["n_sel"], np.int32)).cuda()
    scale = 1.0 / math.sqrt(w.head_dim)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse)
    rng = np.random.default_rng(seed)
    dout = torch.from_numpy(rng.standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16).cuda()
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.full(kc.shape, SENTINEL, dtype=torch.float32, device="cuda")
    dv = torch.full(vc.shape, SENTINEL, dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn_bwd(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse, dout, delta, dq, dk, dv)
    torch.cuda.synchronize()
    hs = list(range(w.heads)) if heads_checked is None else heads_checked
    want = O.attention_grad(x["q"][:, hs], x["k_cache"][:, hs], x["v_cache"][:, hs], x["frame_slot"],
                            s["sel_blocks"][:, hs], s["n_sel"][:, hs], dout.float().cpu().numpy()[:, hs],
                            w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames, scale)
    named = sorted(set(int(v) for v in x["frame_slot"]))
    unnamed = [sl for sl in range(w.cache_slots) if sl not in named]
    dkn, dvn = dk.cpu().numpy()[:, hs], dv.cpu().numpy()[:, hs]
    _check("dq", dq.cpu().numpy()[:, hs], want["dq"])
    _check("dk", dkn[:, :, named], want["dk_cache"][:, :, named])
    _check("dv", dvn[:, :, named], want["dv_cache"][:, :, named])
    if unnamed:
        assert np.all(dkn[:, :, unnamed] == SENTINEL) and np.all(dvn[:, :, unnamed] == SENTINEL)
    # delta is rowsum(dout * out) of the GPU's own bf16 out
    dref = np.sum(dout.float().cpu().numpy() * out.float().cpu().numpy(), axis=-1)
    np.testing.assert_allclose(delta.cpu().numpy(), dref, rtol=1e-4, atol=1e-4)


def _odd(d, T, b, Fc=2, Fh=4, H=2, kf=2, kb=2, n_sink=1, slots=None):
    return I.Workload(name=f"bwd_{d}_{T}_{b}_{Fh}", batch=1, heads=H, head_dim=d, grid=(1, T), block=b,
                      chunk_frames=Fc, hist_frames=Fh, n_sink=n_sink if Fh > 0 else 0,
                      cache_slots=slots if slots is not None else Fh + Fc + 2, dtype="bf16", k_frames=kf,
                      k_blocks=kb, sparsity=float("nan"), seed=9, dist="normal", chunk_index=4)


@pytest.mark.parametrize("d,T,b", [(64, 40, 16), (128, 130, 64), (128, 200, 128), (64, 77, 32), (128, 64, 64)])
def test_backward_odd_geometries(d, T, b):
    _run(_odd(d, T, b))


def test_backward_empty_history():
    _run(_odd(128, 100, 64, Fh=0))


def test_backward_wan480p_shape_two_heads():
    """The 480p chunk's shapes (T=1560, b=64, Fc=3, Fh=6, 80%) on unit-normal inputs; heads 0-1 checked."""
    _run(I.WAN480P_CHUNK.replace(dist="normal", seed=11), heads_checked=[0, 1])


def test_backward_many_heads_every_head_checked():
    """16 heads, 6 history frames of 4 blocks: the history pass's 384 workgroups span all 8 XCD ranges of
    its longest-first launch order, and every head is compared."""
    _run(_odd(128, 128, 32, Fc=2, Fh=6, H=16, kf=3, kb=2))


def test_backward_skewed_selection():
    """Most query blocks name the same three history blocks and a few name their own: history tiles seen
    by almost every query block beside tiles seen by one or none, so the launch order reorders heavily.
    (Each list ascending, without repeats, within the selection's capacity.)"""
    def skew(w, s):
        sel = np.full_like(s["sel_blocks"], -1)
        n = np.zeros_like(s["n_sel"])
        nb, nblk = w.blocks_per_frame, w.hist_frames * w.blocks_per_frame
        for b in range(sel.shape[0]):
            for h in range(sel.shape[1]):
                for qb in range(sel.shape[2]):
                    ids = [0, 1, 2] if (qb + h) % 5 else [(3 + 7 * qb + h) % nblk, (5 + 11 * qb) % nblk]
                    ids = sorted(set(ids))[:sel.shape[3]]
                    sel[b, h, qb, :len(ids)] = ids
                    n[b, h, qb] = len(ids)
        assert nb >= 3
        return {**s, "sel_blocks": sel, "n_sel": n}

    _run(_odd(128, 256, 64, Fc=2, Fh=5, H=8, kf=2, kb=2), sel_fn=skew)


def test_backward_two_batches():
    """B = 2, 5 heads: the history pass's launch order and the key workgroups span (batch, head) pairs of
    both batches; every head of both is compared."""
    _run(_odd(128, 130, 64, Fc=2, Fh=5, H=5, kf=2, kb=2).replace(batch=2, name="bwd_b2"))


def test_backward_selection_lists_near_lf_max_sel():
    """508 selected history blocks per query block (254 frames, 2 of 4 blocks each)."""
    _run(_odd(128, 256, 64, Fc=1, Fh=254, H=1, kf=254, kb=2, n_sink=0, slots=255).replace(chunk_index=300))


def test_backward_is_deterministic():
    """No atomics: two calls on the same inputs give the same bits (480p shape, two heads)."""
    w = I.WAN480P_CHUNK.replace(heads=2, dist="normal", seed=13, name="wan480p_h2")
    x = I.make_inputs(w)
    g = lf.geom_of(w)
    q, kc, vc = P.device_inputs(w, x)
    bufs = lf.Buffers(g, w.k_frames, w.k_blocks, with_lse=True)
    scale = 1.0 / math.sqrt(w.head_dim)
    lf.hsa_attention(g, q, kc, vc, x["frame_slot"], bufs, scale)
    dout = torch.from_numpy(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32)).to(
        torch.bfloat16).cuda()
    res = []
    for _ in range(2):
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        dk = torch.zeros(kc.shape, dtype=torch.float32, device="cuda")
        dv = torch.zeros(kc.shape, dtype=torch.float32, device="cuda")
        lf.lf_block_sparse_attn_bwd(g, q, kc, vc, x["frame_slot"], bufs.sel_blocks, bufs.n_sel, scale, bufs.out,
                                    bufs.lse, dout, delta, dq, dk, dv)
        torch.cuda.synchronize()
        res.append((dq.cpu(), dk.cpu(), dv.cpu()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
