"""CPU oracle for Light Forcing's hierarchical sparse attention (HSA) and its
chunk-aware growth (CAG) budget.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library
and its Python binding) never calls it, and it shares no code with that path:
it is a slow, plain restatement of what the pages define, in float64.

What it follows (Light Forcing, arXiv 2602.04789):
  * technical summary 2.2 "Hierarchical sparse attention": token compression
    by mean pooling of queries and keys at block and frame granularity;
    two-stage mask selection (frames by inner product with frame-level keys,
    then blocks inside each chosen frame with block-level keys); attention only
    on the chosen frame-block pairs.
  * press summary section 3 (hierarchical sparse attention): queries are
    compressed per block, history keys per block and per frame; frame choice
    per query block by inner-product similarity; block choice inside each
    chosen frame; a block-level mask drives the sparse attention kernel.
  * technical summary 2.1 "Chunk-aware growth": s_i = s_base - alpha_i * beta,
    alpha_i scaling as 1/sqrt of the chunk's noise level, beta tuned to meet
    the target sparsity; earlier (cleaner) chunks get the denser budget.
  * Self Forcing page, rolling KV cache paragraph (keep the last L frames,
    evict the oldest) and Rolling Forcing page, dual-cache paragraph (first
    frames kept as a global anchor plus recent frames).

Readings where the pages leave a step open (each restated at its function):
  R1 blocks are cut per frame, ceil(T/b) of them, the last one ragged;
  R2 the frame-level key is the mean over all tokens of the frame;
  R3 queries are pooled per block only;
  R4 block top-k is taken separately inside each chosen frame;
  R5 selection is per (batch, head, query block);
  R6 the current chunk sees all of its own tokens (chunk-granular causality);
  R7 softmax scale 1/sqrt(d), a parameter;
  R8 sink frames are always attended in full and are not top-k candidates;
  R15 ties in a top-k go to the lowest index;
  R18 the single-level ("1D") ablation variant ranks all non-sink history
      blocks in one top-k;
  R19 the backward pass is the gradient of the loss sum(out * dout) through
      the same masks (the selection itself is not differentiated);
  R20 the FP8 variant takes queries and keys as OCP E4M3 codes with one OCP
      MX (E8M0) scale per 32 consecutive channels of each token (per-token
      activation scaling, in the form the matrix cores apply); values and
      P stay bf16.
Pooling sums in float64 and rounds the mean once to float32; scores are
float64 dot products of those float32 values; attention is float64 dense
masked softmax.

Parity pins: every function here is checked by tests against closed forms,
brute force or library routines (see the tests named in each docstring).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Partition (reading R1)
# ---------------------------------------------------------------------------

def block_ranges(tokens_per_frame: int, block: int) -> List[Tuple[int, int]]:
    """Token ranges [start, end) of the blocks of one frame.

    Blocks never straddle frames (blocks are chosen *inside* frames, press
    summary section 3); ceil(T/b) blocks, the last holding the remainder.
    Pinned by tests/test_oracle_compress.py (arithmetic-progression means).
    """
    n = -(-tokens_per_frame // block)
    return [(j * block, min((j + 1) * block, tokens_per_frame)) for j in range(n)]


# ---------------------------------------------------------------------------
# Token compression (technical summary 2.2, "token compression")
# ---------------------------------------------------------------------------

def mean_pool(tokens: np.ndarray) -> np.ndarray:
    """Mean of a [n, d] token set: float64 sum, divided by n, rounded once to float32."""
    total = np.asarray(tokens, dtype=np.float64).sum(axis=0)
    return (total / tokens.shape[0]).astype(np.float32)


def compress(q: np.ndarray, k_cache: np.ndarray, frame_slot: Sequence[int], tokens_per_frame: int,
             block: int, chunk_frames: int, hist_frames: int) -> Dict[str, np.ndarray]:
    """Block-mean queries, block- and frame-mean history keys.

    q        [B, H, chunk_frames*T, d]   current chunk queries
    k_cache  [B, H, S, T, d]             key cache; logical frame f lives in slot frame_slot[f]
    returns  q_blk [B,H,chunk_frames*nb,d], k_blk [B,H,hist_frames*nb,d], k_frm [B,H,hist_frames,d]
    Query block qb = (frame qb // nb, block qb % nb) of the current chunk (R3).
    Frame key = mean over all T tokens of the frame (R2).
    Pinned by tests/test_oracle_compress.py.
    """
    B, H, _, d = q.shape
    T = tokens_per_frame
    ranges = block_ranges(T, block)
    nb = len(ranges)
    q_blk = np.zeros((B, H, chunk_frames * nb, d), np.float32)
    k_blk = np.zeros((B, H, hist_frames * nb, d), np.float32)
    k_frm = np.zeros((B, H, hist_frames, d), np.float32)
    for b in range(B):
        for h in range(H):
            for fc in range(chunk_frames):
                for j, (s, e) in enumerate(ranges):
                    q_blk[b, h, fc * nb + j] = mean_pool(q[b, h, fc * T + s:fc * T + e])
            for f in range(hist_frames):
                frame = k_cache[b, h, frame_slot[f]]
                for j, (s, e) in enumerate(ranges):
                    k_blk[b, h, f * nb + j] = mean_pool(frame[s:e])
                k_frm[b, h, f] = mean_pool(frame)
    return {"q_blk": q_blk, "k_blk": k_blk, "k_frm": k_frm}


# ---------------------------------------------------------------------------
# Two-stage mask selection (technical summary 2.2, "two-stage mask selection")
# ---------------------------------------------------------------------------

def top_k_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores; ties go to the lowest index (R15).

    A full stable sort on the negated scores, then the first k.
    Pinned by tests/test_oracle_select.py (brute-force subset enumeration).
    """
    order = np.argsort(-np.asarray(scores, dtype=np.float64), kind="stable")
    return order[:k]


def effective_k(hist_frames: int, n_sink: int, blocks_per_frame: int, k_frames: int, k_blocks: int) -> Tuple[int, int]:
    """k clamped to what exists: frames to the non-sink history, blocks to a frame."""
    return max(0, min(k_frames, hist_frames - n_sink)), max(0, min(k_blocks, blocks_per_frame))


def max_selected(hist_frames: int, n_sink: int, blocks_per_frame: int, k_frames: int, k_blocks: int) -> int:
    kf, kb = effective_k(hist_frames, n_sink, blocks_per_frame, k_frames, k_blocks)
    return min(n_sink, hist_frames) * blocks_per_frame + kf * kb


def select(q_blk: np.ndarray, k_blk: np.ndarray, k_frm: np.ndarray, hist_frames: int, n_sink: int,
           blocks_per_frame: int, k_frames: int, k_blocks: int) -> Dict[str, np.ndarray]:
    """Frame top-k, then block top-k inside each chosen frame, per query block.

    For query block qb (R5):
      1. frame score s_f = <q_blk[qb], k_frm[f]> (float64) for non-sink frames
         f = n_sink .. hist_frames-1; keep the k_frames best (R15, R8);
      2. in each chosen frame f, block score s_fj = <q_blk[qb], k_blk[f*nb+j]>;
         keep the k_blocks best per frame (R4);
      3. the selected logical block ids are every block of the sink frames
         plus the chosen (f, j) pairs, id = f*nb + j, sorted ascending.
    Returns sel_frames [B,H,nqb,kf] (chosen non-sink frames, ascending),
    sel_blocks [B,H,nqb,max_sel] (padded with -1), n_sel [B,H,nqb], and the
    frame/block scores for tie analysis.
    Pinned by tests/test_oracle_select.py (brute force, plants, invariants).
    """
    B, H, nqb, d = q_blk.shape
    nb = blocks_per_frame
    kf, kb = effective_k(hist_frames, n_sink, nb, k_frames, k_blocks)
    ns = min(n_sink, hist_frames)
    m = ns * nb + kf * kb
    sel_frames = np.full((B, H, nqb, max(kf, 0)), -1, np.int32)
    sel_blocks = np.full((B, H, nqb, max(m, 1)), -1, np.int32)
    n_sel = np.zeros((B, H, nqb), np.int32)
    frame_scores = np.zeros((B, H, nqb, max(hist_frames - ns, 0)), np.float64)
    block_scores = np.full((B, H, nqb, hist_frames, nb), np.nan, np.float64)
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                qv = q_blk[b, h, qb].astype(np.float64)
                cands = list(range(ns, hist_frames))
                fs = np.array([np.dot(qv, k_frm[b, h, f].astype(np.float64)) for f in cands], np.float64)
                frame_scores[b, h, qb] = fs
                chosen = sorted(cands[i] for i in top_k_desc(fs, kf)) if kf > 0 else []
                sel_frames[b, h, qb, :len(chosen)] = chosen
                ids = [f * nb + j for f in range(ns) for j in range(nb)]
                for f in chosen:
                    bs = np.array([np.dot(qv, k_blk[b, h, f * nb + j].astype(np.float64)) for j in range(nb)])
                    block_scores[b, h, qb, f] = bs
                    ids += [f * nb + int(j) for j in top_k_desc(bs, kb)]
                ids = sorted(ids)
                n_sel[b, h, qb] = len(ids)
                sel_blocks[b, h, qb, :len(ids)] = ids
    return {"sel_frames": sel_frames, "sel_blocks": sel_blocks, "n_sel": n_sel,
            "frame_scores": frame_scores, "block_scores": block_scores}


def max_selected_1d(hist_frames: int, n_sink: int, blocks_per_frame: int, k_total: int) -> int:
    ns = min(n_sink, hist_frames)
    return ns * blocks_per_frame + max(0, min(k_total, (hist_frames - ns) * blocks_per_frame))


def select_blocks(q_blk: np.ndarray, k_blk: np.ndarray, hist_frames: int, n_sink: int, blocks_per_frame: int,
                  k_total: int) -> Dict[str, np.ndarray]:
    """Single-level ("1D") selection: one top-k over every non-sink history block.

    The ablation baseline of the press summary, section 4 (ablation
    paragraph): block sparse attention without the frame stage. Reading R18:
    the candidates are all blocks of the non-sink history frames, scored
    <q_blk[qb], k_blk[id]> in float64 exactly as in select(); the k_total best
    are kept (ties to the lowest id, R15), k_total clamped to the candidate
    count; sink frames are attended in full (R8); ids ascending. With
    k_total = k_frames * k_blocks both variants spend the same block budget.
    Pinned by tests/test_oracle_select.py (brute force, a plant the frame
    stage cannot follow, the all-blocks limit).
    """
    B, H, nqb, d = q_blk.shape
    nb = blocks_per_frame
    ns = min(n_sink, hist_frames)
    cands = list(range(ns * nb, hist_frames * nb))
    k = max(0, min(k_total, len(cands)))
    m = ns * nb + k
    sel_blocks = np.full((B, H, nqb, max(m, 1)), -1, np.int32)
    n_sel = np.zeros((B, H, nqb), np.int32)
    scores = np.zeros((B, H, nqb, len(cands)), np.float64)
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                qv = q_blk[b, h, qb].astype(np.float64)
                sc = np.array([np.dot(qv, k_blk[b, h, i].astype(np.float64)) for i in cands], np.float64)
                scores[b, h, qb] = sc
                ids = list(range(ns * nb)) + sorted(cands[int(i)] for i in top_k_desc(sc, k))
                n_sel[b, h, qb] = len(ids)
                sel_blocks[b, h, qb, :len(ids)] = ids
    return {"sel_blocks": sel_blocks, "n_sel": n_sel, "scores": scores}


# ---------------------------------------------------------------------------
# Block-sparse attention (technical summary 2.2, "execution")
# ---------------------------------------------------------------------------

def visible_keys(sel_ids: Sequence[int], tokens_per_frame: int, block: int, hist_frames: int,
                 chunk_frames: int) -> np.ndarray:
    """Boolean mask over the logical key sequence seen by one query block.

    Logical keys: history frames 0..hist_frames-1, then the current chunk's
    frames, T tokens each. A query sees the tokens of its selected history
    blocks and every token of the current chunk (R6).
    """
    T = tokens_per_frame
    ranges = block_ranges(T, block)
    nb = len(ranges)
    mask = np.zeros((hist_frames + chunk_frames) * T, bool)
    for bid in sel_ids:
        if bid < 0:
            continue
        f, j = divmod(int(bid), nb)
        s, e = ranges[j]
        mask[f * T + s:f * T + e] = True
    mask[hist_frames * T:] = True
    return mask


def logical_sequence(cache: np.ndarray, frame_slot: Sequence[int], n_frames: int) -> np.ndarray:
    """Concatenate the cache frames in logical order: [n_frames*T, d] float64."""
    return np.concatenate([np.asarray(cache[frame_slot[f]], np.float64) for f in range(n_frames)], axis=0)


def masked_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float):
    """Dense masked softmax attention in float64 (the plain definition).

    S = scale * q k^T; masked entries -> -inf; P = softmax over keys (row max
    subtracted); O = P v. Returns O [n, d], lse [n] (natural log of the
    row normaliser, including the max), P [n, L].
    Pinned by tests/test_oracle_attention.py (library SDPA, naive loops,
    row sums, convex hull, shift invariance).
    """
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    s = np.where(mask[None, :], s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    l = p.sum(axis=1, keepdims=True)
    p = p / l
    o = p @ np.asarray(v, np.float64)
    lse = (mx + np.log(l))[:, 0]
    return o, lse, p


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, frame_slot: Sequence[int],
              sel_blocks: np.ndarray, n_sel: np.ndarray, tokens_per_frame: int, block: int,
              chunk_frames: int, hist_frames: int, scale: float, qblocks=None) -> Dict[str, np.ndarray]:
    """Block-sparse attention of the current chunk over the cache.

    For each (batch, head, query block) the rows of that block attend to the
    keys ``visible_keys`` allows, through dense masked softmax.
    ``qblocks`` optionally restricts the work to a list of (b, h, qb) triples;
    rows outside it are left as NaN.
    Returns out [B,H,Lq,d] float64 and lse [B,H,Lq] float64.
    """
    B, H, Lq, d = q.shape
    T = tokens_per_frame
    ranges = block_ranges(T, block)
    nb = len(ranges)
    nqb = chunk_frames * nb
    out = np.full((B, H, Lq, d), np.nan)
    lse = np.full((B, H, Lq), np.nan)
    if qblocks is None:
        qblocks = [(b, h, qb) for b in range(B) for h in range(H) for qb in range(nqb)]
    cache_kv = {}
    for (b, h, qb) in qblocks:
        if (b, h) not in cache_kv:
            n_frames = hist_frames + chunk_frames
            cache_kv = {(b, h): (logical_sequence(k_cache[b, h], frame_slot, n_frames),
                                 logical_sequence(v_cache[b, h], frame_slot, n_frames))}
        K, V = cache_kv[(b, h)]
        fc, j = divmod(qb, nb)
        s, e = ranges[j]
        rows = slice(fc * T + s, fc * T + e)
        ids = sel_blocks[b, h, qb, :n_sel[b, h, qb]]
        mask = visible_keys(ids, T, block, hist_frames, chunk_frames)
        o, l, _ = masked_softmax_attention(q[b, h, rows], K, V, mask, scale)
        out[b, h, rows] = o
        lse[b, h, rows] = l
    return {"out": out, "lse": lse}


def masked_softmax_attention_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float,
                                  dout: np.ndarray):
    """Gradients of ``masked_softmax_attention`` for the loss sum(O * dout), float64.

    Chain rule through O = P v, P = softmax(S) row-wise, S = scale q k^T with
    masked entries fixed at -inf:
      dV = P^T dO;   dP = dO v^T;   D_i = sum_j P_ij dP_ij (= dO_i . O_i);
      dS = P * (dP - D);   dq = scale dS k;   dk = scale dS^T q.
    Masked entries have P = 0, so they pass no gradient. Returns dq [n, d],
    dk [L, d], dv [L, d].
    Pinned by tests/test_oracle_backward.py (central finite differences of
    the forward oracle, autograd of an independent torch formulation, and
    the sum rules sum_j dk_j = 0, sum_j dv_j = sum_i dO_i).
    """
    o, _, p = masked_softmax_attention(q, k, v, mask, scale)
    dout = np.asarray(dout, np.float64)
    dv = p.T @ dout
    dp = dout @ np.asarray(v, np.float64).T
    dd = np.sum(dout * o, axis=1, keepdims=True)
    ds = p * (dp - dd)
    dq = scale * (ds @ np.asarray(k, np.float64))
    dk = scale * (ds.T @ np.asarray(q, np.float64))
    return dq, dk, dv


def attention_grad(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, frame_slot: Sequence[int],
                   sel_blocks: np.ndarray, n_sel: np.ndarray, dout: np.ndarray, tokens_per_frame: int, block: int,
                   chunk_frames: int, hist_frames: int, scale: float) -> Dict[str, np.ndarray]:
    """Backward of ``attention`` for the loss sum(out * dout) (the gradient a
    sparse fine-tuning step needs; the press summary's ablation paragraph,
    section 4, compares the sparse attention with and without fine-tuning).

    Each query block contributes through its own mask; key and value
    gradients of one cache row add up over every query block that sees it.
    Rows of cache slots that ``frame_slot`` does not name get zero.
    Returns dq [B,H,Lq,d], dk_cache and dv_cache [B,H,S,T,d], float64.
    """
    B, H, Lq, d = q.shape
    S = k_cache.shape[2]
    T = tokens_per_frame
    ranges = block_ranges(T, block)
    nb = len(ranges)
    nqb = chunk_frames * nb
    n_frames = hist_frames + chunk_frames
    dq = np.zeros((B, H, Lq, d))
    dk_cache = np.zeros((B, H, S, T, d))
    dv_cache = np.zeros((B, H, S, T, d))
    for b in range(B):
        for h in range(H):
            K = logical_sequence(k_cache[b, h], frame_slot, n_frames)
            V = logical_sequence(v_cache[b, h], frame_slot, n_frames)
            dK = np.zeros_like(K)
            dV = np.zeros_like(V)
            for qb in range(nqb):
                fc, j = divmod(qb, nb)
                s, e = ranges[j]
                rows = slice(fc * T + s, fc * T + e)
                ids = sel_blocks[b, h, qb, :n_sel[b, h, qb]]
                mask = visible_keys(ids, T, block, hist_frames, chunk_frames)
                gq, gk, gv = masked_softmax_attention_grad(q[b, h, rows], K, V, mask, scale, dout[b, h, rows])
                dq[b, h, rows] = gq
                dK += gk
                dV += gv
            for f in range(n_frames):
                dk_cache[b, h, frame_slot[f]] = dK[f * T:(f + 1) * T]
                dv_cache[b, h, frame_slot[f]] = dV[f * T:(f + 1) * T]
    return {"dq": dq, "dk_cache": dk_cache, "dv_cache": dv_cache}


# ---------------------------------------------------------------------------
# FP8 inputs (reading R20): OCP 8-bit floating point E4M3 values with OCP
# microscaling (MX) E8M0 scales, one per 32 consecutive channels of a token
# ---------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of OCP E4M3 codes (the variant without infinities), float64.

    Bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa. Exponent
    field 0: subnormal, (m/8) * 2^-6; otherwise (1 + m/8) * 2^(e-7). The one
    NaN pattern per sign is exponent 15 with mantissa 7; the largest finite
    magnitude is 448 (exponent 15, mantissa 6).
    Pinned by tests/test_oracle_fp8.py (printed values, torch's float8_e4m3fn).
    """
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """OCP MX scale: 2^(code - 127); code 255 is NaN. Float64."""
    c = np.asarray(codes, np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """x[..., d] = e4m3(codes[..., d]) * e8m0(scales[..., d // block]), float64.

    codes [..., D] uint8, scales [..., D // block] uint8 (one per block of
    consecutive channels of each token).
    """
    x = e4m3_decode(codes)
    sc = np.repeat(e8m0_decode(scales), block, axis=-1)
    return x * sc


def attention_fp8(q8: np.ndarray, q_scale: np.ndarray, k8_cache: np.ndarray, k_scale: np.ndarray,
                  v_cache: np.ndarray, frame_slot: Sequence[int], sel_blocks: np.ndarray, n_sel: np.ndarray,
                  tokens_per_frame: int, block: int, chunk_frames: int, hist_frames: int, scale: float,
                  qblocks=None) -> Dict[str, np.ndarray]:
    """The block-sparse attention on MX-FP8 queries and keys: the exact values
    the codes and scales stand for, then ``attention`` (float64)."""
    return attention(mx_dequantize(q8, q_scale), mx_dequantize(k8_cache, k_scale), v_cache, frame_slot,
                     sel_blocks, n_sel, tokens_per_frame, block, chunk_frames, hist_frames, scale, qblocks)


# ---------------------------------------------------------------------------
# Chunk-aware growth (technical summary 2.1)
# ---------------------------------------------------------------------------

def round_half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


def ceil_tol(x: float) -> int:
    """ceil with a 1e-9 allowance, so 3.0000000000000004 counts as 3."""
    return int(math.ceil(x - 1e-9))


def chunk_budget(sigma: Sequence[float], weight: Sequence[float], dense: Sequence[bool], s_base: float,
                 s_target: float, hist_frames: Sequence[int], n_sink: Sequence[int], blocks_per_frame: int,
                 k_frames_min: int) -> Dict[str, object]:
    """Per-chunk sparsity s_i = s_base - beta / sqrt(sigma_i) and the top-k sizes it implies.

    alpha_i = 1/sqrt(sigma_i): the adjustment falls with the chunk's noise
    level as a square root, so cleaner (earlier) chunks get lower sparsity.
    beta makes the weighted mean of s_i over the non-dense chunks equal
    s_target:
        sum_i w_i (s_base - beta/sqrt(sigma_i)) = s_target sum_i w_i
        => beta = (s_base - s_target) sum_i w_i / sum_i (w_i / sqrt(sigma_i)).
    Dense chunks get s_i = 0 and no selection.
    Top-k sizing of chunk i (history of F_i frames, n_bpf blocks each, n_s sinks):
        budget_i = (1 - s_i) * F_i * n_bpf - n_s * n_bpf   blocks beyond the sinks
        k_f = min(F_i - n_s, max(k_frames_min, ceil(budget_i / n_bpf)))
        k_b = min(n_bpf, max(1, round_half_up(budget_i / k_f)))
    Pinned by tests/test_oracle_budget.py (mean constraint, monotonicity,
    uniform special case, block-count accounting).
    """
    n = len(sigma)
    sparse = [i for i in range(n) if not dense[i]]
    if sparse:
        num = sum(weight[i] for i in sparse)
        den = sum(weight[i] / math.sqrt(sigma[i]) for i in sparse)
        beta = (s_base - s_target) * num / den
    else:
        beta = 0.0
    s = [0.0] * n
    kf = [0] * n
    kb = [0] * n
    for i in range(n):
        F = hist_frames[i]
        cand = max(F - n_sink[i], 0)
        if dense[i]:
            # every history block attended: the full k
            s[i] = 0.0
            kf[i] = cand
            kb[i] = blocks_per_frame if cand > 0 else 0
            continue
        s[i] = s_base - beta / math.sqrt(sigma[i])
        budget = (1.0 - s[i]) * F * blocks_per_frame - n_sink[i] * blocks_per_frame
        if cand == 0 or budget <= 0:
            kf[i], kb[i] = 0, 0
            continue
        kf[i] = min(cand, max(k_frames_min, ceil_tol(budget / blocks_per_frame)))
        kb[i] = min(blocks_per_frame, max(1, round_half_up(budget / kf[i])))
    return {"beta": beta, "sparsity": s, "k_frames": kf, "k_blocks": kb}


# ---------------------------------------------------------------------------
# KV cache slot table (Self Forcing rolling cache; Rolling Forcing anchors)
# ---------------------------------------------------------------------------

def simulate_cache(policy: str, cache_slots: int, n_sink: int, chunk_frames: int, chunk_index: int):
    """Replay frame-by-frame caching up to the start of chunk ``chunk_index``.

    A slot list is filled as frames are produced; once full, the oldest
    non-anchor frame is evicted and its slot reused (rolling: no anchors;
    anchored: the first n_sink frames are never evicted). Room for the
    current chunk's frames is made the same way, so the returned table is
    (history frames ascending, then the current chunk's frames) with the
    slot each occupies. Returns (absolute frame ids, slots).
    """
    anchors = n_sink if policy == "anchored" else 0
    occupant = [None] * cache_slots  # slot -> absolute frame
    resident: List[int] = []  # absolute frames, oldest first
    total = (chunk_index + 1) * chunk_frames
    for a in range(total):
        free = [s for s in range(cache_slots) if occupant[s] is None]
        if free:
            slot = free[0]
        else:
            victim = next(x for x in resident if x >= anchors)
            slot = occupant.index(victim)
            resident.remove(victim)
        occupant[slot] = a
        resident.append(a)
    frames = sorted(resident)
    slots = [occupant.index(a) for a in frames]
    return frames, slots
