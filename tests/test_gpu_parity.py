"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test draws seeded inputs, runs lf_compress / lf_select /
lf_block_sparse_attn on the GPU and the oracle on the CPU, and compares:
pooled vectors bit-exact, selected ids bit-exact up to score ties within
1e-5 relative, attention (given the oracle's mask) within max-abs 2e-2,
mean-abs 2e-3 and relative L2 1e-2. Pooling and selection are compared on
every query block of every workload; attention on every query block of the
480p chunk, the long-history case and every rollout chunk at step 0, and on
the wide-head case on every head (its first and last three query blocks plus
spread ones).
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


def _full_check(w, x=None, k_frames=None, k_blocks=None, all_rows=False, n_random=4, scale_mult=1.0,
                every_head=False):
    k_frames = w.k_frames if k_frames is None else k_frames
    k_blocks = w.k_blocks if k_blocks is None else k_blocks
    _say(f"[parity] {w.name} B={w.batch} H={w.heads} d={w.head_dim} T={w.tokens_per_frame} b={w.block} "
         f"Fh={w.hist_frames} kf={k_frames} kb={k_blocks} dtype={w.dtype}")
    x = I.make_inputs(w) if x is None else x
    g, dev, bufs = P.gpu_compress_select(w, x, k_frames, k_blocks)
    c, s = P.oracle_compress_select(w, x, k_frames, k_blocks)
    P.assert_pooled_bit_exact(bufs, c)
    n, excused, bad = P.compare_selection(w, bufs, s, k_frames, k_blocks)
    assert not bad, f"{len(bad)} of {n} selections differ without a tie, first: {bad[0]}"
    scale = scale_mult / math.sqrt(w.head_dim)
    qbs = ([(b, h, qb) for b in range(w.batch) for h in range(w.heads) for qb in range(w.n_qblocks)]
           if all_rows else (P.sample_every_head(w) if every_head else P.sample_qblocks(w, n_random)))
    out, lse = P.gpu_attention(w, g, dev, x, s["sel_blocks"], s["n_sel"], scale)
    stats = P.compare_attention(w, x, out, lse, s["sel_blocks"], s["n_sel"], scale, qbs)
    _say(f"[parity] {w.name}: selections {n} ({excused} tie-excused), attention {stats}")
    # The pipeline's own selection drives the same kernel to the same output.
    if excused == 0:
        torch.cuda.synchronize()
        lf.lf_block_sparse_attn(g, *dev, x["frame_slot"], bufs.sel_blocks, bufs.n_sel, scale, bufs.out, bufs.lse)
        torch.cuda.synchronize()
        assert np.array_equal(bufs.out.float().cpu().numpy(), out)
    return x, bufs, s


def test_tiny_fp32_all_rows():
    _full_check(I.TINY_FP32, all_rows=True)


@pytest.mark.parametrize("name", [I.WAN480P_CHUNK.name, I.LONG_HISTORY_SINK.name])
def test_full_size_workloads_every_row(name):
    _full_check(I.WORKLOADS[name], all_rows=True)


def test_wide_head_every_head():
    _full_check(I.WIDE_HEAD, every_head=True)


def test_wan480p_unit_normal_logits():
    """Same shapes with N(0,1) inputs: logits of std ~1, so the softmax is far from uniform."""
    _full_check(I.WAN480P_CHUNK.replace(dist="normal", seed=11), all_rows=True)


@pytest.mark.parametrize("chunk,step", [(c, 0) for c in range(7)] + [(3, 3), (6, 1)])
def test_chunk_rollout(chunk, step):
    r = I.CHUNK_ROLLOUT
    n = r.n_chunks
    bud = lf.lf_chunk_budget(r.sigmas(), None, [True] + [False] * (n - 1), r.s_base, r.s_target,
                             [r.chunk_frames * i for i in range(n)], None, r.blocks_per_frame, r.k_frames_min)
    kf, kb = bud["k_frames"][chunk], bud["k_blocks"][chunk]
    x = I.rollout_chunk_inputs(r, chunk, step, k_frames=kf, k_blocks=kb)
    _full_check(x.pop("workload"), x=x, k_frames=kf, k_blocks=kb, all_rows=(step == 0), n_random=3)


def test_planted_structure_is_recovered():
    """Wide-head low-rank keys: wherever the latent frame gap is large, the true top frames are chosen.
    Long-history plant: the sink is always attended and recent frames favour their diagonal block."""
    w = I.WIDE_HEAD
    x = I.make_inputs(w)
    g, dev, bufs = P.gpu_compress_select(w, x, w.k_frames, w.k_blocks)
    fr = bufs.sel_frames.cpu().numpy()
    a, c = x["frame_factor"][:, :, :w.hist_frames], x["query_factor"]
    lat = np.einsum("bhqr,bhfr->bhqf", c, a)
    top = np.sort(lat, axis=-1)[..., ::-1]
    gap = top[..., w.k_frames - 1] - top[..., w.k_frames]
    # score noise ~ |a_f| * 0.5 / sqrt(tokens in the query block); |a_f| ~ sqrt(8)
    counts = np.array([P.qblock_rows(w, qb).stop - P.qblock_rows(w, qb).start for qb in range(w.n_qblocks)])
    sigma = math.sqrt(8.0) * 0.5 / np.sqrt(counts)
    strong = gap > 6.0 * math.sqrt(2.0) * sigma[None, None, :]
    want = np.sort(np.argsort(-lat, axis=-1, kind="stable")[..., :w.k_frames], axis=-1)
    assert strong.sum() > 100
    assert np.array_equal(fr[strong], want[strong])

    w2 = I.LONG_HISTORY_SINK
    x2 = I.make_inputs(w2)
    g2, dev2, b2 = P.gpu_compress_select(w2, x2, w2.k_frames, w2.k_blocks)
    sel, n_sel = b2.sel_blocks.cpu().numpy(), b2.n_sel.cpu().numpy()
    nb = w2.blocks_per_frame
    assert np.all(sel[..., :nb] == np.arange(nb))
    hits = total = 0
    for h in range(w2.heads):
        for qb in range(w2.n_qblocks):
            fc, j = divmod(qb, nb)
            f = w2.hist_frames - 3 + fc
            ids = set(sel[0, h, qb, :n_sel[0, h, qb]].tolist())
            if any(i // nb == f for i in ids):
                total += 1
                hits += (f * nb + j) in ids
    assert total > 0 and hits == total


@pytest.mark.parametrize("dtype,d,T,b", [("bf16", 64, 100, 48), ("f32", 128, 200, 64), ("bf16", 128, 130, 128),
                                         ("f32", 64, 77, 16), ("bf16", 64, 40, 8), ("bf16", 128, 200, 64),
                                         ("bf16", 128, 90, 40), ("bf16", 128, 250, 96), ("bf16", 64, 300, 128),
                                         ("bf16", 128, 70, 32)])
def test_odd_geometries(dtype, d, T, b):
    w = I.Workload(name=f"odd_{dtype}_{d}_{T}_{b}", batch=2, heads=3, head_dim=d, grid=(1, T), block=b,
                   chunk_frames=2, hist_frames=5, n_sink=1, cache_slots=8, dtype=dtype, k_frames=2, k_blocks=2,
                   sparsity=float("nan"), seed=5, dist="normal", chunk_index=4)
    _full_check(w, all_rows=True)


@pytest.mark.parametrize("dtype,b,mult", [("bf16", 64, 4.0), ("bf16", 64, 16.0), ("bf16", 128, 16.0),
                                          ("f32", 64, 16.0)])
def test_sharp_logits(dtype, b, mult):
    """Logits of std `mult` (unit-normal q and k, scale mult/sqrt(d)). At std 16 the maximum over the
    whole key set sits some 20 above the maximum of the first tile, so the running maximum is overtaken
    by more than 2^16 in probability and the kernel must take its exact rescaling branch, in both the
    single-tile-buffered (b=64, bf16) and the double-buffered kernels."""
    w = I.Workload(name=f"sharp_{dtype}_{b}_{mult:g}", batch=1, heads=4, head_dim=128, grid=(6, 20), block=b,
                   chunk_frames=3, hist_frames=9, n_sink=1, cache_slots=12, dtype=dtype, k_frames=4, k_blocks=2,
                   sparsity=float("nan"), seed=21, dist="normal", chunk_index=3)
    _full_check(w, all_rows=True, scale_mult=mult)


def test_dense_selection_equals_full_attention():
    w = I.TINY_FP32.replace(dtype="bf16", seed=3)
    x = I.make_inputs(w)
    _full_check(w, x=x, k_frames=w.hist_frames, k_blocks=w.blocks_per_frame, all_rows=True)


def test_empty_history_and_empty_selection():
    w = I.WAN480P_CHUNK.replace(hist_frames=0, chunk_index=0, cache_slots=3, seed=7)
    _full_check(w, n_random=4)
    w2 = I.TINY_FP32.replace(seed=9)
    _full_check(w2, k_frames=0, k_blocks=0, all_rows=True)


def test_ignored_ids_and_extra_capacity():
    """Ids of -1 or out of range, and slots past n_sel, do not change the output."""
    w = I.TINY_FP32.replace(dtype="bf16", seed=4)
    x = I.make_inputs(w)
    g, dev, bufs = P.gpu_compress_select(w, x, w.k_frames, w.k_blocks)
    c, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    scale = 1.0 / math.sqrt(w.head_dim)
    base, _ = P.gpu_attention(w, g, dev, x, s["sel_blocks"], s["n_sel"], scale)
    m = s["sel_blocks"].shape[-1]
    noisy = np.full(s["sel_blocks"].shape[:-1] + (m + 6,), 10 ** 6, np.int32)
    noisy[..., 1:m + 1] = s["sel_blocks"]
    noisy[..., 0] = -1
    noisy[..., m + 1] = w.hist_frames * w.blocks_per_frame  # one past the last id
    got, _ = P.gpu_attention(w, g, dev, x, noisy, s["n_sel"] + 2, scale)
    assert np.array_equal(got, base)


def test_duplicate_frames_tie_to_lowest_index():
    w = I.TINY_FP32.replace(dtype="bf16", seed=6)
    x = I.make_inputs(w)
    sl = x["frame_slot"]
    x["k_cache"][:, :, sl[2]] = x["k_cache"][:, :, sl[1]]  # frames 1 and 2 identical
    x["k_cache"][:, :, sl[3]] = x["k_cache"][:, :, sl[1]]
    _, bufs, s = _full_check(w, x=x, k_frames=1, k_blocks=2, all_rows=True)
    fr = bufs.sel_frames.cpu().numpy()[..., 0]
    assert not np.any((fr == 2) | (fr == 3))


def test_many_frames_and_blocks_limits():
    w = I.Workload(name="limits_frames250_blocks500", batch=1, heads=1, head_dim=64, grid=(1, 16), block=16,
                   chunk_frames=1, hist_frames=249, n_sink=2, cache_slots=250, dtype="bf16", k_frames=5, k_blocks=1,
                   sparsity=float("nan"), seed=8, dist="normal", chunk_index=249)
    _full_check(w, all_rows=True)
    w2 = I.Workload(name="limits_blocks500", batch=1, heads=2, head_dim=64, grid=(1, 8000), block=16,
                    chunk_frames=1, hist_frames=2, n_sink=0, cache_slots=3, dtype="bf16", k_frames=1, k_blocks=70,
                    sparsity=float("nan"), seed=9, dist="normal", chunk_index=2)
    _full_check(w2, n_random=3)


@pytest.mark.parametrize("d,T,b,Fh,kb", [(64, 128, 16, 128, 4), (128, 256, 64, 254, 2)])
def test_selection_lists_at_lf_max_sel(d, T, b, Fh, kb):
    """Every query block selects LF_MAX_SEL (512) or 508 history blocks (every frame, half of its blocks):
    the longest walks the kernels take, in the double-buffered (b = 16) and single-stage (b = 64) walks."""
    w = I.Workload(name=f"maxsel_d{d}_b{b}", batch=1, heads=1, head_dim=d, grid=(1, T), block=b, chunk_frames=1,
                   hist_frames=Fh, n_sink=0, cache_slots=Fh + 1, dtype="bf16", k_frames=Fh, k_blocks=kb,
                   sparsity=float("nan"), seed=12, dist="normal", chunk_index=Fh)
    assert lf.lf_max_sel(lf.geom_of(w), Fh, kb) in (lf.LF_MAX_SEL, lf.LF_MAX_SEL - 4)
    _full_check(w, all_rows=True)


@pytest.mark.parametrize("dtype,H,Fh", [("f32", 16, 8), ("f32", 2, 3), ("bf16", 24, 12)])
def test_pooling_launch_shapes(dtype, H, Fh):
    """The pooling launch splits frames into column slices only when that grid gives every workgroup a
    compute unit of its own, else pools whole frames. Both shapes must give the oracle's bits: (f32, 16
    heads, 8 frames) is 512 float32 frame slices, beyond the chip's 256 compute units, so whole frames;
    (f32, 2 heads, 3 frames) takes slices; (bf16, 24 heads, 12 frames) whole frames again."""
    w = I.Workload(name=f"poolshape_{dtype}_h{H}_f{Fh}", batch=1, heads=H, head_dim=128, grid=(1, 200), block=64,
                   chunk_frames=1, hist_frames=Fh, n_sink=0, cache_slots=Fh + 1, dtype=dtype, k_frames=2,
                   k_blocks=2, sparsity=float("nan"), seed=14, dist="normal", chunk_index=Fh)
    _full_check(w, all_rows=True)
