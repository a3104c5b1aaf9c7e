"""Pool-on-commit and the fused per-step selection (Light Forcing technical
summary 2.2; the Self Forcing page's rolling cache keeps committed frames
unchanged until eviction, so their pooled keys can be computed once).

Checks: pooled keys by slot are bit-exact against the oracle's pooling of the
same frames; slots not named are not written; lf_select_fused equals
lf_compress + lf_select bit for bit and the oracle's selection.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf
from oracle import lf_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _pooled_cache(w, g, kc, slots):
    S, nb, d = w.cache_slots, w.blocks_per_frame, w.head_dim
    kp_blk = torch.full((w.batch, w.heads, S, nb, d), float("nan"), dtype=torch.float32, device="cuda")
    kp_frm = torch.full((w.batch, w.heads, S, d), float("nan"), dtype=torch.float32, device="cuda")
    lf.lf_pool_keys(g, kc, slots, kp_blk, kp_frm)
    torch.cuda.synchronize()
    return kp_blk, kp_frm


@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_pool_keys_bit_exact_by_slot(name):
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    g = lf.geom_of(w)
    q, kc, vc = P.device_inputs(w, x)
    hist_slots = [int(s) for s in x["frame_slot"][:w.hist_frames]]
    kp_blk, kp_frm = _pooled_cache(w, g, kc, hist_slots)
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames,
                   w.hist_frames)
    nb = w.blocks_per_frame
    kb_np, kf_np = kp_blk.cpu().numpy(), kp_frm.cpu().numpy()
    for f, s in enumerate(hist_slots):
        assert np.array_equal(kb_np[:, :, s].view(np.uint32),
                              c["k_blk"][:, :, f * nb:(f + 1) * nb].view(np.uint32)), f"blocks of frame {f}"
        assert np.array_equal(kf_np[:, :, s].view(np.uint32), c["k_frm"][:, :, f].view(np.uint32)), f"frame {f}"
    others = [s for s in range(w.cache_slots) if s not in hist_slots]
    assert np.isnan(kb_np[:, :, others]).all() and np.isnan(kf_np[:, :, others]).all()


@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_fused_select_equals_compress_then_select(name):
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    g, dev, bufs = P.gpu_compress_select(w, x, w.k_frames, w.k_blocks)
    q, kc, vc = dev
    kp_blk, kp_frm = _pooled_cache(w, g, kc, [int(s) for s in x["frame_slot"][:w.hist_frames]])
    fused = lf.Buffers(g, w.k_frames, w.k_blocks)
    lf.lf_select_fused(g, q, kp_blk, kp_frm, x["frame_slot"], w.k_frames, w.k_blocks, fused.sel_frames,
                       fused.sel_blocks, fused.n_sel, q_blk=fused.q_blk)
    torch.cuda.synchronize()
    for a, b in ((fused.sel_blocks, bufs.sel_blocks), (fused.n_sel, bufs.n_sel), (fused.sel_frames, bufs.sel_frames)):
        assert torch.equal(a, b)
    assert torch.equal(fused.q_blk.view(torch.int32), bufs.q_blk.view(torch.int32))
    c, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    checked, excused, bad = P.compare_selection(w, fused, s, w.k_frames, w.k_blocks)
    print(f"[fused] {name}: {checked} query blocks, {excused} excused ties", flush=True)
    assert not bad, bad[:3]


def test_fused_select_over_a_rolling_rollout():
    """Commit each chunk's frames once, then select for the next chunk from
    the pooled cache: every chunk's selection equals the oracle's."""
    ro = I.CHUNK_ROLLOUT
    for i in (1, 3, 6):
        w = ro.chunk_workload(i, 3, 4)
        x = I.make_inputs(w)
        g = lf.geom_of(w)
        q, kc, vc = P.device_inputs(w, x)
        kp_blk, kp_frm = _pooled_cache(w, g, kc, [int(s) for s in x["frame_slot"][:w.hist_frames]])
        bufs = lf.Buffers(g, w.k_frames, w.k_blocks)
        lf.lf_select_fused(g, q, kp_blk, kp_frm, x["frame_slot"], w.k_frames, w.k_blocks, bufs.sel_frames,
                           bufs.sel_blocks, bufs.n_sel)
        torch.cuda.synchronize()
        c, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
        checked, excused, bad = P.compare_selection(w, bufs, s, w.k_frames, w.k_blocks)
        assert not bad, (i, bad[:3])
