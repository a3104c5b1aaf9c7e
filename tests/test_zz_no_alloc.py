"""The allocation-free backward entry point (lf_block_sparse_attn_bwd_noalloc).

Its row scratch is a fixed device array of the library instead of a caller
buffer; otherwise it runs the same kernels as lf_block_sparse_attn_bwd, whose
results are deterministic, so the two must agree bit for bit. Two calls in a
row on different workloads, the second smaller, check that nothing of the
first call's scratch leaks into the second. The size limit is checked on the
host, before any device work.
"""
import ctypes
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_lf_amd import inputs as I
from block_sparse_attention_lf_amd import lf
from oracle import lf_oracle as O
from tests import parity as P

SENTINEL = 777.0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_rows_beyond_the_scratch_are_refused_before_any_device_work():
    w = I.TINY_FP32.replace(dtype="bf16", heads=4, grid=(1, (lf.LF_NOALLOC_MAX_ROWS // 4) + 1))
    g = lf.geom_of(w)
    st = lf.lib().lf_block_sparse_attn_bwd_noalloc(ctypes.byref(g), None, None, None, None, None, None, 0,
                                                   ctypes.c_float(0.1), None, None, None, None, None, None, None)
    assert st == -2  # LF_ERR_GEOM
    assert b"LF_NOALLOC_MAX_ROWS" in lf.lib().lf_last_error()


def _grads(w, seed):
    x = I.make_inputs(w)
    g = lf.geom_of(w)
    q, kc, vc = P.device_inputs(w, x)
    _, s = P.oracle_compress_select(w, x, w.k_frames, w.k_blocks)
    sb = torch.from_numpy(np.ascontiguousarray(s["sel_blocks"], np.int32)).cuda()
    ns = torch.from_numpy(np.ascontiguousarray(s["n_sel"], np.int32)).cuda()
    scale = 1.0 / math.sqrt(w.head_dim)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse)
    rng = np.random.default_rng(seed)
    dout = torch.from_numpy(rng.standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16).cuda()

    def bufs():
        return (torch.empty(q.shape, dtype=torch.float32, device="cuda"),
                torch.full(kc.shape, SENTINEL, dtype=torch.float32, device="cuda"),
                torch.full(kc.shape, SENTINEL, dtype=torch.float32, device="cuda"))

    ref, got = bufs(), bufs()
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lf.lf_block_sparse_attn_bwd(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse, dout, delta, *ref)
    lf.lf_block_sparse_attn_bwd_noalloc(g, q, kc, vc, x["frame_slot"], sb, ns, scale, out, lse, dout, *got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.gpu
def test_noalloc_backward_equals_the_workspace_backward_twice_in_a_row():
    big = I.WAN480P_CHUNK.replace(heads=4, seed=31)
    small = I.TINY_FP32.replace(dtype="bf16", seed=32)
    for w, seed in ((big, 5), (small, 6)):
        _say(f"[noalloc] {w.name} H={w.heads} T={w.tokens_per_frame} b={w.block} rows={w.batch * w.heads * w.q_len}")
        ref, got = _grads(w, seed)
        for name, a, b in zip(("dq", "dk_cache", "dv_cache"), ref, got):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert np.all(np.isfinite(b)), name
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
