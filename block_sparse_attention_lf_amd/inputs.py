"""Seeded synthetic workloads for Light Forcing's hierarchical sparse attention.

This module only *draws* inputs: shapes, seeds and value distributions of the
workloads the attention path is measured and tested on. It holds none of the
method's arithmetic (no pooling, scoring, selection, softmax or budgeting), so
that the GPU path and the CPU oracle can both be fed from it without sharing
any computation.

Source pages:
  * Light Forcing (arXiv 2602.04789), technical summary section 2.2 "HSA":
    queries and keys are pooled per block and per frame, frames then blocks
    are selected, attention runs on the chosen frame-block pairs.
  * Self Forcing news page, rolling KV cache paragraph: the cache keeps the
    last L frames and evicts the oldest one.
  * Rolling Forcing page, section 3 "dual cache": the first frames are kept
    as a global anchor next to a window of recent frames.

All floating point tensors are returned as numpy float32 arrays. For bf16
workloads every value is already rounded to bf16 (round to nearest even), so
the float32 array holds exactly the numbers the GPU sees; ``bf16_bits``
gives the matching uint16 payload.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# Cache policies understood by the frame-slot planner.
POLICY_ROLLING = 0
POLICY_ANCHORED = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call's geometry plus the recipe of its synthetic inputs.

    Frame = ``tokens_per_frame`` tokens (a ``grid`` latent image). Frames are
    cut into ``block``-token blocks per frame; the last block of a frame holds
    the remainder. The current chunk has ``chunk_frames`` frames of queries;
    the cache holds ``hist_frames`` history frames (the first ``n_sink`` of
    them pinned as attention sinks) plus the current chunk's own keys/values.
    ``k_frames``/``k_blocks`` are the two top-k sizes; ``sparsity`` is the
    fraction of history blocks left out that they were sized for.
    """

    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple
    block: int
    chunk_frames: int
    hist_frames: int
    n_sink: int
    cache_slots: int
    dtype: str  # "f32" or "bf16"
    k_frames: int
    k_blocks: int
    sparsity: float
    seed: int
    dist: str  # recipe name, see make_inputs
    policy: int = POLICY_ROLLING
    chunk_index: int = 0  # index of the chunk being generated (drives the slot table)

    @property
    def tokens_per_frame(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def blocks_per_frame(self) -> int:
        return -(-self.tokens_per_frame // self.block)

    @property
    def q_len(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def n_qblocks(self) -> int:
        return self.chunk_frames * self.blocks_per_frame

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny fp32 case: 8x8 latent grid, 16-token blocks, one query frame against a
# history of four frames; keep two frames, then two blocks in each.
TINY_FP32 = Workload(
    name="tiny_fp32_h2_d64_t64_b16", batch=1, heads=2, head_dim=64, grid=(8, 8), block=16,
    chunk_frames=1, hist_frames=4, n_sink=0, cache_slots=5, dtype="f32",
    k_frames=2, k_blocks=2, sparsity=0.75, seed=0, dist="normal", chunk_index=7)

# Wan-1.3B-like 480p chunk: 30x52 latent grid (1560 tokens per frame), three
# query frames (4680 queries), six history frames in a rolling nine-slot cache.
# 80% of the 150 history blocks are skipped: 30 = 3 frames x 10 blocks.
WAN480P_CHUNK = Workload(
    name="wan480p_chunk_h12_d128_t1560_b64_hist6", batch=1, heads=12, head_dim=128, grid=(30, 52),
    block=64, chunk_frames=3, hist_frames=6, n_sink=0, cache_slots=9, dtype="bf16",
    k_frames=3, k_blocks=10, sparsity=0.80, seed=1, dist="normal_scaled", chunk_index=4)

# Long history: 21 history frames + the current 3-frame chunk (37440 keys),
# frame 0 pinned as an attention sink in an anchored cache. 90% sparsity:
# 0.1 x 525 = 52.5 blocks; the sink takes 25, 27.5 / 3 frames -> 9 blocks each,
# 25 + 27 = 52 of 525 selected.
LONG_HISTORY_SINK = Workload(
    name="long_history_sink_h12_d128_t1560_b64_hist21", batch=1, heads=12, head_dim=128,
    grid=(30, 52), block=64, chunk_frames=3, hist_frames=21, n_sink=1, cache_slots=24,
    dtype="bf16", k_frames=3, k_blocks=9, sparsity=0.90, seed=2, dist="planted_sink_diag",
    policy=POLICY_ANCHORED, chunk_index=9)

# Wide heads: 40 heads, 45x80 latent grid (3600 tokens per frame), 128-token
# blocks, nine history frames. 85% sparsity: 0.15 x 261 = 39.15 -> 3 x 13 = 39.
WIDE_HEAD = Workload(
    name="wide_head_h40_d128_t3600_b128_hist9", batch=1, heads=40, head_dim=128, grid=(45, 80),
    block=128, chunk_frames=3, hist_frames=9, n_sink=0, cache_slots=12, dtype="bf16",
    k_frames=3, k_blocks=13, sparsity=0.85, seed=4, dist="lowrank", chunk_index=5)


@dataclasses.dataclass(frozen=True)
class Rollout:
    """Chunk-wise autoregressive rollout: chunk i attends to every earlier chunk.

    Chunk 0 has no history and runs dense. Each chunk is denoised in
    ``steps`` steps with fresh queries per step; its keys/values are drawn
    once, at its first step, and stay in the cache afterwards. The per-chunk
    sparsity follows chunk-aware growth with noise levels ``sigma`` linear
    from ``sigma_lo`` to ``sigma_hi``.
    """

    name: str = "chunk_rollout_7x3_h12_d128_t1560_b64"
    n_chunks: int = 7
    steps: int = 4
    heads: int = 12
    head_dim: int = 128
    grid: tuple = (30, 52)
    block: int = 64
    chunk_frames: int = 3
    dtype: str = "bf16"
    s_base: float = 0.9
    s_target: float = 0.8
    sigma_lo: float = 0.1
    sigma_hi: float = 1.0
    k_frames_min: int = 3
    seed: int = 3

    @property
    def tokens_per_frame(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def blocks_per_frame(self) -> int:
        return -(-self.tokens_per_frame // self.block)

    def sigmas(self) -> List[float]:
        n = self.n_chunks
        return [self.sigma_lo + (self.sigma_hi - self.sigma_lo) * i / (n - 1) for i in range(n)]

    def chunk_workload(self, i: int, k_frames: int, k_blocks: int) -> Workload:
        return Workload(
            name=f"{self.name}_chunk{i}", batch=1, heads=self.heads, head_dim=self.head_dim,
            grid=self.grid, block=self.block, chunk_frames=self.chunk_frames,
            hist_frames=self.chunk_frames * i, n_sink=0,
            cache_slots=self.chunk_frames * self.n_chunks, dtype=self.dtype,
            k_frames=k_frames, k_blocks=k_blocks, sparsity=float("nan"), seed=self.seed * 1000 + i,
            dist="normal", chunk_index=i)


CHUNK_ROLLOUT = Rollout()

WORKLOADS: Dict[str, Workload] = {w.name: w for w in (TINY_FP32, WAN480P_CHUNK, LONG_HISTORY_SINK, WIDE_HEAD)}


# --------------------------------------------------------------------------
# bf16 helpers (bit manipulation only)
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 payload of float32 values that are already exactly bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------
# FP8 inputs: OCP E4M3 codes with an OCP MX (E8M0) scale per 32 channels
# --------------------------------------------------------------------------

def mx_quantize(x: np.ndarray, block: int = 32):
    """Quantise float values to E4M3 codes with one E8M0 scale per ``block``
    consecutive channels of the last axis: the shared exponent of a block is
    the smallest one with max |x| / 2^exp <= 448 (E4M3's largest value, so no
    element clips), elements are x / 2^exp rounded to nearest-even E4M3. An
    all-zero block gets scale 2^-127. Returns (codes uint8 [..., D], scales uint8 [..., D/block]).
    (Input preparation for the FP8 variant; the kernel and the oracle only
    read the codes.)
    """
    import torch  # float8_e4m3fn gives nearest-even rounding of the scaled values

    x = np.asarray(x, np.float32)
    D = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (D // block, block)).astype(np.float64)
    amax = np.max(np.abs(xb), axis=-1)
    exp = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), -127).astype(np.int64)
    exp = np.clip(exp, -127, 127)
    y = np.clip(xb / np.exp2(exp)[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.reshape(x.shape).copy(), (exp + 127).astype(np.uint8)


# --------------------------------------------------------------------------
# Cache slot tables (which physical slot holds which logical frame)
# --------------------------------------------------------------------------

def rotated_slots(w: Workload) -> np.ndarray:
    """A slot table as a rolling/anchored ring would leave it at ``w.chunk_index``.

    Absolute frame a (0-based over the whole video) lives in slot
      rolling : a mod S
      anchored: a for the first n_sink frames, else n_sink + (a - n_sink) mod (S - n_sink).
    The history is the most recent frames that fit next to the current chunk
    (plus the anchors); logical frame order is ascending absolute frame index,
    history first, then the current chunk.
    This mirrors the caches on the pages; it is input bookkeeping, not
    attention arithmetic.
    """
    S, F_c, F_h, ns = w.cache_slots, w.chunk_frames, w.hist_frames, w.n_sink
    first_cur = w.chunk_index * F_c
    if w.policy == POLICY_ANCHORED:
        recent = F_h - ns
        frames = list(range(ns)) + list(range(first_cur - recent, first_cur))
    else:
        frames = list(range(first_cur - F_h, first_cur))
    frames += list(range(first_cur, first_cur + F_c))
    assert all(a >= 0 for a in frames), "history longer than the frames generated so far"

    def slot(a: int) -> int:
        if w.policy == POLICY_ANCHORED:
            return a if a < ns else ns + (a - ns) % (S - ns)
        return a % S

    slots = np.array([slot(a) for a in frames], dtype=np.int32)
    assert len(set(slots.tolist())) == len(slots)
    return slots


# --------------------------------------------------------------------------
# Value recipes
# --------------------------------------------------------------------------

def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(w: Workload, seed: Optional[int] = None, q_seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw q [B,H,Lq,d], k_cache/v_cache [B,H,S,T,d] and the slot table.

    Recipes (``w.dist``):
      normal            q, k, v ~ N(0, 1)
      normal_scaled     q, k, v ~ N(0, 1) / sqrt(d)
      planted_sink_diag N(0,1)/sqrt(d) plus a plant on the keys: every token
                        of history frame 0 gets one shared offset vector whose
                        elements are +-2 sigma (seeded signs, sigma = 1/sqrt(d));
                        history frame F_h-3+j gets + q of current frame j at the
                        same spatial token (a diagonal boost), j = 0..2.
      lowrank           an orthonormal 8 x d basis A; per frame a_f ~ N(0, I8),
                        per query block c ~ N(0, I8); k = a_f A + N(0, 0.5^2),
                        q = c A + N(0, 0.5^2), v ~ N(0, 1). The true top frames of
                        a query block are the top of c . a_f.
    Slots not named in the table are filled with the same distribution (they
    are stale cache content and must never be read).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, H, d, T, S = w.batch, w.heads, w.head_dim, w.tokens_per_frame, w.cache_slots
    Lq = w.q_len
    slots = rotated_slots(w)
    out: Dict[str, np.ndarray] = {"frame_slot": slots}
    extra: Dict[str, np.ndarray] = {}

    if w.dist in ("normal", "normal_scaled", "planted_sink_diag"):
        std = 1.0 / math.sqrt(d) if w.dist != "normal" else 1.0
        k = _normal(rng, (B, H, S, T, d), std)
        v = _normal(rng, (B, H, S, T, d), std)
        q = _normal(rng if q_seed is None else np.random.default_rng(q_seed), (B, H, Lq, d), std)
        if w.dist == "planted_sink_diag":
            sigma = np.float32(1.0 / math.sqrt(d))
            signs = rng.integers(0, 2, size=(B, H, 1, d)).astype(np.float32) * 2 - 1
            offset = 2 * sigma * signs
            k[:, :, slots[0]] += offset
            F_h = w.hist_frames
            for j in range(min(3, w.chunk_frames, F_h)):
                f = F_h - 3 + j
                if f < w.n_sink:
                    continue
                k[:, :, slots[f]] += q[:, :, j * T:(j + 1) * T]
            extra["sink_offset"] = offset.reshape(B, H, d)
    elif w.dist == "lowrank":
        r = 8
        g = rng.standard_normal(size=(d, r))
        basis, _ = np.linalg.qr(g)  # d x r, orthonormal columns
        A = basis.T.astype(np.float32)  # r x d, orthonormal rows
        n_frames = w.hist_frames + w.chunk_frames
        a = rng.standard_normal(size=(B, H, S, r)).astype(np.float32)
        k = np.einsum("bhsr,rd->bhsd", a, A)[:, :, :, None, :] + _normal(rng, (B, H, S, T, d), 0.5)
        v = _normal(rng, (B, H, S, T, d), 1.0)
        nqb = w.n_qblocks
        c = rng.standard_normal(size=(B, H, nqb, r)).astype(np.float32)
        cq = np.einsum("bhqr,rd->bhqd", c, A)
        q = _normal(rng, (B, H, Lq, d), 0.5)
        nb = w.blocks_per_frame
        for qb in range(nqb):
            fc, j = divmod(qb, nb)
            s0 = fc * T + j * w.block
            e0 = fc * T + min((j + 1) * w.block, T)
            q[:, :, s0:e0] += cq[:, :, qb][:, :, None, :]
        extra["basis"] = A
        extra["frame_factor"] = a[:, :, slots[:n_frames]]  # logical frame order
        extra["query_factor"] = c
    else:
        raise ValueError(f"unknown recipe {w.dist}")

    out["q"] = _finish(q, w.dtype)
    out["k_cache"] = _finish(k, w.dtype)
    out["v_cache"] = _finish(v, w.dtype)
    out.update(extra)
    return out


def rollout_chunk_inputs(r: Rollout, i: int, step: int, kv_prev: Optional[Dict[str, np.ndarray]] = None,
                         k_frames: int = 0, k_blocks: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of chunk ``i``, denoise step ``step`` of the rollout.

    Keys/values of chunk i are drawn at its first step and reused for the
    later steps (pass the previous step's dict as ``kv_prev``); queries are
    fresh N(0,1) at every step. The cache holds every earlier chunk: slot of
    absolute frame a is a (no eviction: all 21 frames fit).
    """
    w = r.chunk_workload(i, k_frames, k_blocks)
    B, H, d, T, S = 1, r.heads, r.head_dim, r.tokens_per_frame, w.cache_slots
    if kv_prev is None:
        k = np.zeros((B, H, S, T, d), np.float32)
        v = np.zeros((B, H, S, T, d), np.float32)
        for c in range(i + 1):  # every chunk up to and including i; drawn from its own stream
            rc = np.random.default_rng(r.seed * 1000 + c)
            kc = _normal(rc, (B, H, r.chunk_frames, T, d))
            vc = _normal(rc, (B, H, r.chunk_frames, T, d))
            k[:, :, c * r.chunk_frames:(c + 1) * r.chunk_frames] = kc
            v[:, :, c * r.chunk_frames:(c + 1) * r.chunk_frames] = vc
        k = _finish(k, r.dtype)
        v = _finish(v, r.dtype)
    else:
        k, v = kv_prev["k_cache"], kv_prev["v_cache"]
    qr = np.random.default_rng(r.seed * 1000003 + i * 97 + step + 1)
    q = _finish(_normal(qr, (B, H, w.q_len, d)), r.dtype)
    slots = np.arange(w.hist_frames + w.chunk_frames, dtype=np.int32)
    return {"q": q, "k_cache": k, "v_cache": v, "frame_slot": slots, "workload": w}
