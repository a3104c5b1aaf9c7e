"""GPU tests of lf_check_selection, the debug check of selection lists.

The rule it checks, restated here from include/lf.h: a row (b*H + h)*nqb + qb
is bad when n_sel is outside [0, max_sel], or one of its first n_sel ids is
outside [0, Fh*nb), or an id is not greater than the one before it. The count
and the first bad row are compared with a numpy evaluation of that rule on
the same lists: lf_select's own lists (none bad), and copies with planted
faults of each kind.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _rule(sel: np.ndarray, n_sel: np.ndarray, n_ids: int):
    max_sel = sel.shape[-1]
    sel = sel.reshape(-1, max_sel)
    n_sel = n_sel.reshape(-1)
    bad = []
    for r, n in enumerate(n_sel):
        if n < 0 or n > max_sel:
            bad.append(r)
            continue
        ids = sel[r, :n].astype(np.int64)
        if np.any(ids < 0) or np.any(ids >= n_ids) or np.any(np.diff(ids) <= 0):
            bad.append(r)
    return len(bad), (bad[0] if bad else -1)


def _check(g, sel, n_sel):
    res = torch.full((2,), 12345, dtype=torch.int32, device="cuda")
    lf.lf_check_selection(g, sel, n_sel, res)
    torch.cuda.synchronize()
    return tuple(int(v) for v in res.cpu())


@pytest.mark.parametrize("name", ["tiny_fp32_h2_d64_t64_b16", "wan480p_chunk_h12_d128_t1560_b64_hist6"])
def test_selection_lists_pass_and_planted_faults_are_found(name):
    w = I.WORKLOADS[name]
    _say(f"[check_selection] {name}")
    g = lf.geom_of(w)
    x = I.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, kc, vc = (torch.from_numpy(x[k]).to(dt).cuda() for k in ("q", "k_cache", "v_cache"))
    bufs = lf.Buffers(g, w.k_frames, w.k_blocks)
    lf.lf_compress(g, q, kc, x["frame_slot"], bufs.q_blk, bufs.k_blk, bufs.k_frm)
    lf.lf_select(g, bufs.q_blk, bufs.k_blk, bufs.k_frm, w.k_frames, w.k_blocks, bufs.sel_frames, bufs.sel_blocks,
                 bufs.n_sel)
    torch.cuda.synchronize()
    n_ids = w.hist_frames * w.blocks_per_frame
    assert _check(g, bufs.sel_blocks, bufs.n_sel) == (0, -1)

    sel = bufs.sel_blocks.cpu().numpy().copy()
    n = bufs.n_sel.cpu().numpy().copy()
    flat_sel = sel.reshape(-1, sel.shape[-1])
    flat_n = n.reshape(-1)
    rows = flat_n.shape[0]
    assert flat_n.min() >= 2 and rows >= 8
    plants = {  # row -> fault (five distinct rows)
        rows - 1: "duplicate", 1: "descending", rows // 2: "out_of_range", 2: "too_many", 5: "negative"}
    assert len(plants) == 5
    for r, kind in plants.items():
        if kind == "duplicate":
            flat_sel[r, 1] = flat_sel[r, 0]
        elif kind == "descending":
            flat_sel[r, 0], flat_sel[r, 1] = flat_sel[r, 1], flat_sel[r, 0]
        elif kind == "out_of_range":
            flat_sel[r, flat_n[r] - 1] = n_ids
        elif kind == "too_many":
            flat_n[r] = sel.shape[-1] + 1
        else:
            flat_n[r] = -1
    want = _rule(sel, n, n_ids)
    assert want[0] == len(plants)
    got = _check(g, torch.from_numpy(sel).cuda(), torch.from_numpy(n).cuda())
    _say(f"[check_selection] planted: want {want}, got {got}")
    assert got == want
    # an id past n_sel is not looked at
    sel2 = bufs.sel_blocks.cpu().numpy().copy()
    sel2.reshape(-1, sel2.shape[-1])[0, -1] = -7
    n2 = bufs.n_sel.cpu().numpy().copy()
    n2.reshape(-1)[0] = n2.reshape(-1)[0] - 1
    assert _check(g, torch.from_numpy(sel2).cuda(), torch.from_numpy(n2).cuda()) == _rule(sel2, n2, n_ids)


def test_empty_history_has_no_bad_rows():
    w = I.TINY_FP32.replace(hist_frames=0, cache_slots=1)
    g = lf.geom_of(w)
    n = torch.zeros((w.batch, w.heads, w.n_qblocks), dtype=torch.int32, device="cuda")
    sel = torch.full((w.batch, w.heads, w.n_qblocks, 1), -1, dtype=torch.int32, device="cuda")
    assert _check(g, sel, n) == (0, -1)
