"""The hot path under HIP graph capture.

One call (compress -> select -> block-sparse attention, and the FP8
variant) is captured into a graph with torch.cuda.graph and replayed
several times, with eager work of the program and synchronisations between
the replays; every replay must reproduce the eager results bit for bit.
The path allocates nothing, synchronises nothing and enqueues no memset, so
it can be captured; the slot table and the selection sizes are fixed at
capture time (they are kernel arguments).
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_graph_replay_matches_eager():
    w = I.WAN480P_CHUNK.replace(heads=2, name="wan480p_chunk_h2")
    _say(f"[graph] {w.name}")
    x = I.make_inputs(w)
    g = lf.geom_of(w)
    q, kc, vc = P.device_inputs(w, x)
    slots = x["frame_slot"]
    scale = 1.0 / math.sqrt(w.head_dim)
    bufs = lf.Buffers(g, w.k_frames, w.k_blocks, with_lse=True)
    q8, qs = (torch.from_numpy(a).cuda() for a in I.mx_quantize(x["q"]))
    k8, ks = (torch.from_numpy(a).cuda() for a in I.mx_quantize(x["k_cache"]))
    out8 = torch.empty_like(bufs.out)

    def call(stream):
        lf.hsa_attention(g, q, kc, vc, slots, bufs, scale, stream)
        lf.lf_block_sparse_attn_fp8(g, q8, qs, k8, ks, vc, slots, bufs.sel_blocks, bufs.n_sel, scale, out8, None,
                                    stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = [t.clone() for t in (bufs.q_blk, bufs.k_blk, bufs.k_frm, bufs.sel_blocks, bufs.n_sel, bufs.out, bufs.lse,
                                out8)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (bufs.q_blk, bufs.k_blk, bufs.k_frm, bufs.out, bufs.lse, out8):
            t.zero_()  # eager work between replays; the replay must rewrite everything
        bufs.sel_blocks.fill_(-7)
        bufs.n_sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bufs.q_blk, bufs.k_blk, bufs.k_frm, bufs.sel_blocks, bufs.n_sel, bufs.out, bufs.lse, out8)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"
        _say(f"[graph] replay {rep} matches")
