"""The oracle still reproduces the stored golden fixtures (written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

from block_sparse_attention_lf_amd import inputs as I
from oracle import lf_oracle as O

G = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_selection_golden():
    g = json.load(open(os.path.join(G, "tiny_fp32_selection.json")))
    w = I.TINY_FP32
    x = I.make_inputs(w)
    assert x["frame_slot"].tolist() == g["frame_slot"]
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames)
    s = O.select(c["q_blk"], c["k_blk"], c["k_frm"], w.hist_frames, w.n_sink, w.blocks_per_frame, w.k_frames, w.k_blocks)
    assert s["sel_blocks"].tolist() == g["sel_blocks"] and s["n_sel"].tolist() == g["n_sel"]


def test_rollout_budget_golden():
    g = json.load(open(os.path.join(G, "chunk_rollout_budget.json")))
    r = I.CHUNK_ROLLOUT
    n = r.n_chunks
    out = O.chunk_budget(r.sigmas(), [1.0] * n, [True] + [False] * (n - 1), r.s_base, r.s_target,
                         [r.chunk_frames * i for i in range(n)], [0] * n, r.blocks_per_frame, r.k_frames_min)
    assert abs(out["beta"] - g["beta"]) < 1e-15
    assert out["k_frames"] == g["k_frames"] and out["k_blocks"] == g["k_blocks"]
    np.testing.assert_allclose(out["sparsity"], g["sparsity"], rtol=0, atol=1e-15)
