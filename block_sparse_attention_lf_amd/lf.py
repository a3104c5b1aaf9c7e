"""Thin Python binding of liblf.so (C ABI in include/lf.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory (tensors) and the
stream; this module checks shapes/dtypes, passes raw pointers and raises
``LfError`` on a non-OK status. There is no fallback: if the library is not
built or cannot be loaded, every call raises.

Function names mirror the C entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # noqa: F401  (load torch's HIP runtime first; liblf.so binds to the same libamdhip64)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblf.so")

LF_F32, LF_BF16 = 0, 1
LF_CACHE_ROLLING, LF_CACHE_ANCHORED = 0, 1
LF_MAX_FRAMES, LF_MAX_BLOCKS_PER_FRAME, LF_MAX_BLOCK, LF_MAX_SEL, LF_MAX_CANDIDATES_1D = 256, 512, 128, 512, 4096
LF_NOALLOC_MAX_ROWS = 1 << 20
LF_MAX_CACHE_SLOTS = 16384

STATUS = {0: "LF_OK", -1: "LF_ERR_NULL", -2: "LF_ERR_GEOM", -3: "LF_ERR_DTYPE", -4: "LF_ERR_K",
          -5: "LF_ERR_ALIGN", -6: "LF_ERR_HIP", -7: "LF_ERR_SLOT", -8: "LF_ERR_ARG"}

# Every symbol include/lf.h declares.
EXPORTS = ("lf_compress", "lf_max_sel", "lf_select", "lf_max_sel_1d", "lf_select_blocks", "lf_pool_keys",
           "lf_select_fused", "lf_check_selection", "lf_block_sparse_attn",
           "lf_block_sparse_attn_fp8", "lf_block_sparse_attn_bwd", "lf_block_sparse_attn_bwd_noalloc",
           "lf_chunk_budget", "lf_cache_frame_slots", "lf_status_str", "lf_last_error", "lf_build_id")


class LfError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")
        self.status = status


class lf_geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "heads", "head_dim", "tokens_per_frame", "block",
                                              "chunk_frames", "hist_frames", "n_sink", "cache_slots", "dtype")]

    @property
    def blocks_per_frame(self) -> int:
        return -(-self.tokens_per_frame // self.block)

    @property
    def n_qblocks(self) -> int:
        return self.chunk_frames * self.blocks_per_frame

    @property
    def q_len(self) -> int:
        return self.chunk_frames * self.tokens_per_frame


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_F64P = ctypes.POINTER(ctypes.c_double)


def expected_build_id() -> str:
    """The id a library built from this tree's sources carries."""
    from block_sparse_attention_lf_amd.build import source_hash

    return source_hash()


def lib() -> ctypes.CDLL:
    """Load liblf.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_sparse_attention_lf_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.lf_build_id.restype = ctypes.c_char_p
    L.lf_build_id.argtypes = []
    built, tree = L.lf_build_id().decode(), expected_build_id()
    if built != tree:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (id {built}, tree {tree}); "
                           "run `python -m block_sparse_attention_lf_amd.build`")
    G = ctypes.POINTER(lf_geom)
    sig = {
        "lf_compress": (ctypes.c_int, [G, _P, _P, _I32P, _P, _P, _P, _P]),
        "lf_max_sel": (ctypes.c_int32, [G, ctypes.c_int32, ctypes.c_int32]),
        "lf_select": (ctypes.c_int, [G, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, ctypes.c_int32, _P]),
        "lf_max_sel_1d": (ctypes.c_int32, [G, ctypes.c_int32]),
        "lf_pool_keys": (ctypes.c_int, [G, _P, _I32P, ctypes.c_int32, _P, _P, _P]),
        "lf_select_fused": (ctypes.c_int, [G, _P, _P, _P, _I32P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                           ctypes.c_int32, _P, _P]),
        "lf_select_blocks": (ctypes.c_int, [G, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_int32, _P]),
        "lf_check_selection": (ctypes.c_int, [G, _P, _P, ctypes.c_int32, _P, _P]),
        "lf_block_sparse_attn": (ctypes.c_int, [G, _P, _P, _P, _I32P, _P, _P, ctypes.c_int32, ctypes.c_float,
                                                _P, _P, _P]),
        "lf_block_sparse_attn_fp8": (ctypes.c_int, [G, _P, _P, _P, _P, _P, _I32P, _P, _P, ctypes.c_int32,
                                                    ctypes.c_float, _P, _P, _P]),
        "lf_block_sparse_attn_bwd": (ctypes.c_int, [G, _P, _P, _P, _I32P, _P, _P, ctypes.c_int32, ctypes.c_float,
                                                    _P, _P, _P, _P, _P, _P, _P, _P]),
        "lf_block_sparse_attn_bwd_noalloc": (ctypes.c_int, [G, _P, _P, _P, _I32P, _P, _P, ctypes.c_int32,
                                                            ctypes.c_float, _P, _P, _P, _P, _P, _P, _P]),
        "lf_chunk_budget": (ctypes.c_int, [ctypes.c_int32, _F64P, _F64P, ctypes.POINTER(ctypes.c_uint8),
                                           ctypes.c_double, ctypes.c_double, _I32P, _I32P, ctypes.c_int32,
                                           ctypes.c_int32, _F64P, _F64P, _I32P, _I32P]),
        "lf_cache_frame_slots": (ctypes.c_int, [ctypes.c_int32] * 5 + [_I32P, _I32P, _I32P]),
        "lf_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "lf_last_error": (ctypes.c_char_p, []),
        "lf_build_id": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LfError(status, where, lib().lf_last_error().decode())


def make_geom(batch, heads, head_dim, tokens_per_frame, block, chunk_frames, hist_frames, n_sink, cache_slots,
              dtype) -> lf_geom:
    dt = {"bf16": LF_BF16, "f32": LF_F32, torch.bfloat16: LF_BF16, torch.float32: LF_F32}.get(dtype, dtype)
    return lf_geom(batch, heads, head_dim, tokens_per_frame, block, chunk_frames, hist_frames, n_sink, cache_slots,
                   int(dt))


def geom_of(w) -> lf_geom:
    """lf_geom of an ``inputs.Workload``."""
    return make_geom(w.batch, w.heads, w.head_dim, w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames,
                     w.n_sink, w.cache_slots, w.dtype)


def _slots(frame_slot: Sequence[int]):
    arr = np.ascontiguousarray(np.asarray(frame_slot, dtype=np.int32))
    return arr, arr.ctypes.data_as(_I32P)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} (cuda={t.is_cuda}, contiguous={t.is_contiguous()})")


def _tdtype(g: lf_geom):
    return torch.bfloat16 if g.dtype == LF_BF16 else torch.float32


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def lf_max_sel(g: lf_geom, k_frames: int, k_blocks: int) -> int:
    return int(lib().lf_max_sel(ctypes.byref(g), k_frames, k_blocks))


def lf_compress(g: lf_geom, q, k_cache, frame_slot, q_blk, k_blk, k_frm, stream=None) -> None:
    """Mean-pool query blocks and history key blocks/frames (see include/lf.h)."""
    D, nb = g.head_dim, g.blocks_per_frame
    _need(q, (g.batch, g.heads, g.q_len, D), _tdtype(g), "q")
    _need(k_cache, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), _tdtype(g), "k_cache")
    _need(q_blk, (g.batch, g.heads, g.n_qblocks, D), torch.float32, "q_blk")
    _need(k_blk, (g.batch, g.heads, g.hist_frames * nb, D), torch.float32, "k_blk")
    _need(k_frm, (g.batch, g.heads, g.hist_frames, D), torch.float32, "k_frm")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_compress(ctypes.byref(g), _ptr(q), _ptr(k_cache), sp, _ptr(q_blk), _ptr(k_blk), _ptr(k_frm),
                             _stream(stream)), "lf_compress")


def lf_select(g: lf_geom, q_blk, k_blk, k_frm, k_frames: int, k_blocks: int, sel_frames, sel_blocks, n_sel,
              stream=None) -> None:
    """Frame top-k then per-frame block top-k per query block (see include/lf.h)."""
    D, nb = g.head_dim, g.blocks_per_frame
    _need(q_blk, (g.batch, g.heads, g.n_qblocks, D), torch.float32, "q_blk")
    _need(k_blk, (g.batch, g.heads, g.hist_frames * nb, D), torch.float32, "k_blk")
    _need(k_frm, (g.batch, g.heads, g.hist_frames, D), torch.float32, "k_frm")
    max_sel = sel_blocks.shape[-1]
    _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
    _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    if sel_frames is not None:
        _need(sel_frames, (g.batch, g.heads, g.n_qblocks, k_frames), torch.int32, "sel_frames")
    _check(lib().lf_select(ctypes.byref(g), _ptr(q_blk), _ptr(k_blk), _ptr(k_frm), k_frames, k_blocks,
                           _ptr(sel_frames), _ptr(sel_blocks), _ptr(n_sel), max_sel, _stream(stream)), "lf_select")


def lf_pool_keys(g: lf_geom, k_cache, slots, kp_blk, kp_frm, stream=None) -> None:
    """Pool the frames in the given cache slots into slot-indexed pooled caches (see include/lf.h)."""
    D, nb, S = g.head_dim, g.blocks_per_frame, g.cache_slots
    _need(k_cache, (g.batch, g.heads, S, g.tokens_per_frame, D), _tdtype(g), "k_cache")
    _need(kp_blk, (g.batch, g.heads, S, nb, D), torch.float32, "kp_blk")
    _need(kp_frm, (g.batch, g.heads, S, D), torch.float32, "kp_frm")
    arr = np.ascontiguousarray(np.asarray(slots, np.int32))
    sp = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(lib().lf_pool_keys(ctypes.byref(g), _ptr(k_cache), sp, int(arr.size), _ptr(kp_blk), _ptr(kp_frm),
                              _stream(stream)), "lf_pool_keys")


def lf_select_fused(g: lf_geom, q, kp_blk, kp_frm, frame_slot, k_frames: int, k_blocks: int, sel_frames, sel_blocks,
                    n_sel, q_blk=None, stream=None) -> None:
    """Query pooling + two-stage selection against slot-indexed pooled keys (see include/lf.h)."""
    D, nb, S = g.head_dim, g.blocks_per_frame, g.cache_slots
    _need(q, (g.batch, g.heads, g.q_len, D), _tdtype(g), "q")
    _need(kp_blk, (g.batch, g.heads, S, nb, D), torch.float32, "kp_blk")
    _need(kp_frm, (g.batch, g.heads, S, D), torch.float32, "kp_frm")
    max_sel = sel_blocks.shape[-1]
    _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
    _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    if sel_frames is not None:
        _need(sel_frames, (g.batch, g.heads, g.n_qblocks, k_frames), torch.int32, "sel_frames")
    if q_blk is not None:
        _need(q_blk, (g.batch, g.heads, g.n_qblocks, D), torch.float32, "q_blk")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_select_fused(ctypes.byref(g), _ptr(q), _ptr(kp_blk), _ptr(kp_frm), sp, k_frames, k_blocks,
                                 _ptr(sel_frames), _ptr(sel_blocks), _ptr(n_sel), max_sel, _ptr(q_blk),
                                 _stream(stream)), "lf_select_fused")


def lf_max_sel_1d(g: lf_geom, k_total: int) -> int:
    return int(lib().lf_max_sel_1d(ctypes.byref(g), k_total))


def lf_select_blocks(g: lf_geom, q_blk, k_blk, k_total: int, sel_blocks, n_sel, stream=None) -> None:
    """Single-level ("1D") block top-k over all non-sink history blocks (see include/lf.h)."""
    D, nb = g.head_dim, g.blocks_per_frame
    _need(q_blk, (g.batch, g.heads, g.n_qblocks, D), torch.float32, "q_blk")
    _need(k_blk, (g.batch, g.heads, g.hist_frames * nb, D), torch.float32, "k_blk")
    max_sel = sel_blocks.shape[-1]
    _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
    _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    _check(lib().lf_select_blocks(ctypes.byref(g), _ptr(q_blk), _ptr(k_blk), k_total, _ptr(sel_blocks), _ptr(n_sel),
                                  max_sel, _stream(stream)), "lf_select_blocks")


def lf_check_selection(g: lf_geom, sel_blocks, n_sel, result, stream=None) -> None:
    """Debug check of selection lists (see include/lf.h): result (2 int32, device) gets the number of rows that
    break the invariants and the first such row (-1 if none), on the stream."""
    max_sel = sel_blocks.shape[-1]
    _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
    _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    _need(result, (2,), torch.int32, "result")
    _check(lib().lf_check_selection(ctypes.byref(g), _ptr(sel_blocks), _ptr(n_sel), max_sel, _ptr(result),
                                    _stream(stream)), "lf_check_selection")


def lf_block_sparse_attn(g: lf_geom, q, k_cache, v_cache, frame_slot, sel_blocks, n_sel, softmax_scale: float, out,
                         lse=None, stream=None) -> None:
    """Attention of the current chunk over its selected history blocks + the chunk (see include/lf.h)."""
    D = g.head_dim
    _need(q, (g.batch, g.heads, g.q_len, D), _tdtype(g), "q")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), _tdtype(g), name)
    _need(out, (g.batch, g.heads, g.q_len, D), _tdtype(g), "out")
    if lse is not None:
        _need(lse, (g.batch, g.heads, g.q_len), torch.float32, "lse")
    max_sel = 0 if sel_blocks is None else sel_blocks.shape[-1]
    if sel_blocks is not None:
        _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
        _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_block_sparse_attn(ctypes.byref(g), _ptr(q), _ptr(k_cache), _ptr(v_cache), sp, _ptr(sel_blocks),
                                      _ptr(n_sel), max_sel, float(softmax_scale), _ptr(out), _ptr(lse),
                                      _stream(stream)), "lf_block_sparse_attn")


def lf_block_sparse_attn_fp8(g: lf_geom, q8, q_scale, k8_cache, k_scale, v_cache, frame_slot, sel_blocks, n_sel,
                             softmax_scale: float, out, lse=None, stream=None) -> None:
    """lf_block_sparse_attn on MX-FP8 queries and keys (E4M3 codes + E8M0 scales per 32 channels; see include/lf.h)."""
    D = g.head_dim
    _need(q8, (g.batch, g.heads, g.q_len, D), torch.uint8, "q8")
    _need(q_scale, (g.batch, g.heads, g.q_len, D // 32), torch.uint8, "q_scale")
    kshape = (g.batch, g.heads, g.cache_slots, g.tokens_per_frame)
    _need(k8_cache, kshape + (D,), torch.uint8, "k8_cache")
    _need(k_scale, kshape + (D // 32,), torch.uint8, "k_scale")
    _need(v_cache, kshape + (D,), torch.bfloat16, "v_cache")
    _need(out, (g.batch, g.heads, g.q_len, D), torch.bfloat16, "out")
    if lse is not None:
        _need(lse, (g.batch, g.heads, g.q_len), torch.float32, "lse")
    max_sel = 0 if sel_blocks is None else sel_blocks.shape[-1]
    if sel_blocks is not None:
        _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
        _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_block_sparse_attn_fp8(ctypes.byref(g), _ptr(q8), _ptr(q_scale), _ptr(k8_cache), _ptr(k_scale),
                                          _ptr(v_cache), sp, _ptr(sel_blocks), _ptr(n_sel), max_sel,
                                          float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)),
           "lf_block_sparse_attn_fp8")


def lf_block_sparse_attn_bwd(g: lf_geom, q, k_cache, v_cache, frame_slot, sel_blocks, n_sel, softmax_scale: float,
                             out, lse, dout, delta, dq, dk_cache, dv_cache, stream=None) -> None:
    """Backward of lf_block_sparse_attn (see include/lf.h): float32 dq, dk_cache, dv_cache."""
    D = g.head_dim
    _need(q, (g.batch, g.heads, g.q_len, D), torch.bfloat16, "q")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), torch.bfloat16, name)
    for name, t in (("out", out), ("dout", dout)):
        _need(t, (g.batch, g.heads, g.q_len, D), torch.bfloat16, name)
    for name, t in (("lse", lse), ("delta", delta)):
        _need(t, (g.batch, g.heads, g.q_len), torch.float32, name)
    _need(dq, (g.batch, g.heads, g.q_len, D), torch.float32, "dq")
    for name, t in (("dk_cache", dk_cache), ("dv_cache", dv_cache)):
        _need(t, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), torch.float32, name)
    max_sel = 0 if sel_blocks is None else sel_blocks.shape[-1]
    if sel_blocks is not None:
        _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
        _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_block_sparse_attn_bwd(ctypes.byref(g), _ptr(q), _ptr(k_cache), _ptr(v_cache), sp,
                                          _ptr(sel_blocks), _ptr(n_sel), max_sel, float(softmax_scale), _ptr(out),
                                          _ptr(lse), _ptr(dout), _ptr(delta), _ptr(dq), _ptr(dk_cache),
                                          _ptr(dv_cache), _stream(stream)), "lf_block_sparse_attn_bwd")


def lf_block_sparse_attn_bwd_noalloc(g: lf_geom, q, k_cache, v_cache, frame_slot, sel_blocks, n_sel,
                                     softmax_scale: float, out, lse, dout, dq, dk_cache, dv_cache, stream=None) -> None:
    """lf_block_sparse_attn_bwd with its row scratch in the library's fixed device array (see include/lf.h):
    allocates nothing; calls that overlap on one GPU race."""
    D = g.head_dim
    _need(q, (g.batch, g.heads, g.q_len, D), torch.bfloat16, "q")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), torch.bfloat16, name)
    for name, t in (("out", out), ("dout", dout)):
        _need(t, (g.batch, g.heads, g.q_len, D), torch.bfloat16, name)
    _need(lse, (g.batch, g.heads, g.q_len), torch.float32, "lse")
    _need(dq, (g.batch, g.heads, g.q_len, D), torch.float32, "dq")
    for name, t in (("dk_cache", dk_cache), ("dv_cache", dv_cache)):
        _need(t, (g.batch, g.heads, g.cache_slots, g.tokens_per_frame, D), torch.float32, name)
    max_sel = 0 if sel_blocks is None else sel_blocks.shape[-1]
    if sel_blocks is not None:
        _need(sel_blocks, (g.batch, g.heads, g.n_qblocks, max_sel), torch.int32, "sel_blocks")
        _need(n_sel, (g.batch, g.heads, g.n_qblocks), torch.int32, "n_sel")
    arr, sp = _slots(frame_slot)
    _check(lib().lf_block_sparse_attn_bwd_noalloc(ctypes.byref(g), _ptr(q), _ptr(k_cache), _ptr(v_cache), sp,
                                                  _ptr(sel_blocks), _ptr(n_sel), max_sel, float(softmax_scale),
                                                  _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_cache),
                                                  _ptr(dv_cache), _stream(stream)),
           "lf_block_sparse_attn_bwd_noalloc")


def lf_chunk_budget(sigma, weight, dense, s_base: float, s_target: float, hist_frames, n_sink, blocks_per_frame: int,
                    k_frames_min: int):
    """Chunk-aware growth: per-chunk sparsity and top-k sizes (host only). Returns a dict."""
    n = len(sigma)
    sig = np.ascontiguousarray(sigma, np.float64)
    w = None if weight is None else np.ascontiguousarray(weight, np.float64)
    dn = np.ascontiguousarray(np.asarray(dense, bool).astype(np.uint8))
    hf = np.ascontiguousarray(hist_frames, np.int32)
    ns = None if n_sink is None else np.ascontiguousarray(n_sink, np.int32)
    s = np.zeros(n, np.float64)
    kf = np.zeros(n, np.int32)
    kb = np.zeros(n, np.int32)
    beta = ctypes.c_double(0.0)
    _check(lib().lf_chunk_budget(n, sig.ctypes.data_as(_F64P), None if w is None else w.ctypes.data_as(_F64P),
                                 dn.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), s_base, s_target,
                                 hf.ctypes.data_as(_I32P), None if ns is None else ns.ctypes.data_as(_I32P),
                                 blocks_per_frame, k_frames_min, s.ctypes.data_as(_F64P), ctypes.byref(beta),
                                 kf.ctypes.data_as(_I32P), kb.ctypes.data_as(_I32P)), "lf_chunk_budget")
    return {"beta": beta.value, "sparsity": s.tolist(), "k_frames": kf.tolist(), "k_blocks": kb.tolist()}


def lf_cache_frame_slots(policy: int, cache_slots: int, n_sink: int, chunk_frames: int, chunk_index: int):
    """Slot table of a rolling / anchored cache for one chunk (host only). Returns (hist_frames, slots, frame_ids)."""
    slots = np.zeros(max(cache_slots, 1), np.int32)
    ids = np.zeros(max(cache_slots, 1), np.int32)
    hist = ctypes.c_int32(0)
    _check(lib().lf_cache_frame_slots(policy, cache_slots, n_sink, chunk_frames, chunk_index, ctypes.byref(hist),
                                      slots.ctypes.data_as(_I32P), ids.ctypes.data_as(_I32P)),
           "lf_cache_frame_slots")
    n = hist.value + chunk_frames
    return hist.value, slots[:n].tolist(), ids[:n].tolist()


# --------------------------------------------------------------------------
# Convenience: buffers and the three device steps on one stream
# --------------------------------------------------------------------------

class Buffers:
    """Device buffers of one attention call's intermediates (allocated once, reused)."""

    def __init__(self, g: lf_geom, k_frames: int, k_blocks: int, device="cuda", with_lse: bool = False):
        B, H, D, nb = g.batch, g.heads, g.head_dim, g.blocks_per_frame
        self.k_frames, self.k_blocks = k_frames, k_blocks
        self.max_sel = max(lf_max_sel(g, k_frames, k_blocks), 1)
        f32, i32 = torch.float32, torch.int32
        self.q_blk = torch.empty((B, H, g.n_qblocks, D), dtype=f32, device=device)
        self.k_blk = torch.empty((B, H, g.hist_frames * nb, D), dtype=f32, device=device)
        self.k_frm = torch.empty((B, H, g.hist_frames, D), dtype=f32, device=device)
        self.sel_frames = torch.empty((B, H, g.n_qblocks, k_frames), dtype=i32, device=device)
        self.sel_blocks = torch.empty((B, H, g.n_qblocks, self.max_sel), dtype=i32, device=device)
        self.n_sel = torch.empty((B, H, g.n_qblocks), dtype=i32, device=device)
        self.out = torch.empty((B, H, g.q_len, D), dtype=_tdtype(g), device=device)
        self.lse = torch.empty((B, H, g.q_len), dtype=f32, device=device) if with_lse else None


def hsa_attention(g: lf_geom, q, k_cache, v_cache, frame_slot, bufs: Buffers, softmax_scale: Optional[float] = None,
                  stream=None):
    """One hierarchical sparse attention call: compress -> select -> block-sparse attention."""
    scale = softmax_scale if softmax_scale is not None else 1.0 / float(np.sqrt(g.head_dim))
    lf_compress(g, q, k_cache, frame_slot, bufs.q_blk, bufs.k_blk, bufs.k_frm, stream)
    lf_select(g, bufs.q_blk, bufs.k_blk, bufs.k_frm, bufs.k_frames, bufs.k_blocks, bufs.sel_frames, bufs.sel_blocks,
              bufs.n_sel, stream)
    lf_block_sparse_attn(g, q, k_cache, v_cache, frame_slot, bufs.sel_blocks, bufs.n_sel, scale, bufs.out, bufs.lse,
                         stream)
    return bufs.out
