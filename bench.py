"""Benchmark of one hierarchical sparse attention call per step on one MI355X.

A step is the whole hot path for one (chunk, denoise step, layer): the cache
slot table and chunk budget on the host, then lf_compress -> lf_select ->
lf_block_sparse_attn on the GPU. The workload is the Wan-1.3B-like 480p chunk
(12 heads, d=128, 1560 tokens per frame, 3 query frames, 6 history frames,
64-token blocks, 80% sparsity, bf16). Inputs are synthetic, seeded, and
resident in HBM before timing; four input sets (about 400 MB) rotate from
step to step so each step reads its keys/values cold from HBM, as successive
layers would.

Prints one JSON line. ``value`` is effective attention TFLOP/s of the whole
step (FLOPs actually needed on the selected blocks plus the current chunk,
4*n_q*n_k*d over valid tokens, divided by the step time).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective attention TFLOP/s + % MFMA bf16 peak per 480p chunk; ms/chunk-layer"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
N_SETS = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the 480p chunk)")
    ap.add_argument("--sets", type=int, default=N_SETS,
                    help="input sets rotated over the steps (default 4, together larger than the MALL)")
    ap.add_argument("--path", choices=("step", "fused"), default="step",
                    help="step: compress + select + attention every step (every hot-path row); fused: keys pooled "
                         "once on commit, then fused query pooling + selection and attention per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="also time lf_block_sparse_attn_bwd (bf16) and report it under 'backward'")
    ap.add_argument("--fp8", action="store_true",
                    help="also time lf_block_sparse_attn_fp8 (MX-FP8 q/k) on the same selections; report under 'fp8'")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (by default the long-history and wide-head workloads "
                         "and the 7-chunk x 4-step rollout follow, under 'configs' and 'rollout')")
    ap.add_argument("--cpu-single-thread", action="store_true",
                    help="also time the oracle on one thread on the tiny fp32 case and the 480p chunk")
    ap.add_argument("--cpu-sample-qblocks", type=int, default=0, help="0: every query block (the whole call)")
    ap.add_argument("--dense-vs-sdpa", action="store_true",
                    help="also time dense attention (no history) against torch's scaled_dot_product_attention "
                         "(flash and memory-efficient backends) at the chunk shapes; report under 'dense_vs_sdpa'")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one elementwise kernel that reads and writes this many MiB "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


def effective_flops(w, sel: np.ndarray, n_sel: np.ndarray) -> float:
    """sum over (b, h, query block) of 4 * rows * keys * d, valid tokens only."""
    T, b, nb, d = w.tokens_per_frame, w.block, w.blocks_per_frame, w.head_dim
    blen = np.array([min(b, T - j * b) for j in range(nb)], np.int64)
    qlen = np.tile(blen, w.chunk_frames)  # rows of each query block
    total = 0.0
    for bi in range(w.batch):
        for h in range(w.heads):
            for qb in range(w.n_qblocks):
                ids = sel[bi, h, qb, :n_sel[bi, h, qb]]
                keys = w.q_len + int(blen[ids % nb].sum())
                total += 4.0 * qlen[qb] * keys * d
    return total


def compress_bytes(w) -> float:
    """Algorithmic HBM bytes of lf_compress: read q and the history keys, write the pooled vectors."""
    es = 2 if w.dtype == "bf16" else 4
    B, H, d = w.batch, w.heads, w.head_dim
    read = B * H * (w.q_len + w.hist_frames * w.tokens_per_frame) * d * es
    write = B * H * (w.n_qblocks + w.hist_frames * w.blocks_per_frame + w.hist_frames) * d * 4
    return float(read + write)


def sources_hash(paths) -> str:
    """First 16 hex digits of the sha256 over the files' code, in the given order: C and C++ comments and
    blank lines are dropped and trailing spaces stripped, so an edit of comments alone keeps the hash (the
    kernel it describes is the same)."""
    import re

    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


# The attention kernel's sources: its own file and the headers it includes.
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_lf_amd", "csrc", f)
                for f in ("attention.hip", "mfma.h", "lf_internal.h")]


def traffic_from_profiles(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, if they match this kernel."""
    p = os.path.join(ROOT, "profiles", "attention_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != sources_hash(ATTN_SOURCES) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def rollout(warmup: int):
    """The chunk-wise rollout: chunk i (3 frames) attends to every earlier chunk, 4 denoise steps per chunk
    with fresh queries, keys/values drawn once per chunk; chunk 0 runs dense, chunks 1-6 take the chunk-aware
    budget. Each call (compress + select + attention, plus the host slot table) is timed with HIP events;
    the whole cache (21 frames) is resident. Returns per-chunk and total figures."""
    import torch

    from block_sparse_attention_lf_amd import inputs as I
    from block_sparse_attention_lf_amd import lf

    r = I.CHUNK_ROLLOUT
    n = r.n_chunks
    hist = [r.chunk_frames * i for i in range(n)]
    bud = lf.lf_chunk_budget(r.sigmas(), None, [True] + [False] * (n - 1), r.s_base, r.s_target, hist, None,
                             r.blocks_per_frame, r.k_frames_min)
    full = I.rollout_chunk_inputs(r, n - 1, 0)  # the cache with every chunk's keys/values
    kc = torch.from_numpy(full["k_cache"]).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(full["v_cache"]).to(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(r.head_dim)
    chunks = []
    tot_ms, tot_flops = 0.0, 0.0
    for i in range(n):
        kf, kb = bud["k_frames"][i], bud["k_blocks"][i]
        w = r.chunk_workload(i, kf, kb)
        g = lf.geom_of(w)
        bufs = lf.Buffers(g, kf, kb)
        slots = np.arange(w.hist_frames + w.chunk_frames, dtype=np.int32)
        qs = [torch.from_numpy(I.rollout_chunk_inputs(r, i, st, kv_prev=full)["q"]).to(torch.bfloat16).cuda()
              for st in range(r.steps)]
        for j in range(warmup):
            lf.hsa_attention(g, qs[j % r.steps], kc, vc, slots, bufs, scale, stream)
        torch.cuda.synchronize()
        ms, fl = [], []
        for st in range(r.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lf.hsa_attention(g, qs[st], kc, vc, slots, bufs, scale, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
            fl.append(effective_flops(w, bufs.sel_blocks.cpu().numpy(), bufs.n_sel.cpu().numpy()))
        sel_blocks = int(bufs.n_sel[0, 0, 0].item())
        chunks.append({"chunk": i, "hist_frames": w.hist_frames, "k_frames": kf, "k_blocks": kb,
                       "sparsity": round(float(bud["sparsity"][i]), 4), "blocks_selected_per_qblock": sel_blocks,
                       "ms_per_call": round(float(np.mean(ms)), 4), "effective_gflop_per_call": round(np.mean(fl) / 1e9, 2),
                       "tflops": round(float(np.sum(fl)) / (float(np.sum(ms)) * 1e-3) / 1e12, 1)})
        tot_ms += float(np.sum(ms))
        tot_flops += float(np.sum(fl))
    return {"name": r.name, "calls": n * r.steps, "total_ms": round(tot_ms, 3),
            "total_effective_gflop": round(tot_flops / 1e9, 1),
            "tflops": round(tot_flops / (tot_ms * 1e-3) / 1e12, 1), "beta": round(float(bud["beta"]), 6),
            "chunks": chunks}


def dense_vs_sdpa(warmup: int, steps: int):
    """Dense attention of a chunk over itself (no history: every query block sees every key) through
    lf_block_sparse_attn, beside torch's scaled_dot_product_attention on the same bf16 tensors with only its
    flash and memory-efficient backends enabled. Shapes: the 480p chunk (12 heads, 3 frames of 1560 tokens),
    twice as many frames, and the wide head's 40 heads. HIP events on the current stream, medians."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    from block_sparse_attention_lf_amd import lf

    stream = torch.cuda.current_stream()

    def med_ms(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    rows = []
    for heads, frames, tpf, d in ((12, 3, 1560, 128), (12, 6, 1560, 128), (40, 3, 1560, 128)):
        n = frames * tpf
        flops = 4.0 * n * n * d * heads
        gen = torch.Generator().manual_seed(1234 + heads + frames)
        q, k, v = (torch.randn(1, heads, n, d, generator=gen).to(torch.bfloat16).cuda() for _ in range(3))
        g = lf.make_geom(1, heads, d, tpf, 64, frames, 0, 0, frames, "bf16")
        kc, vc = k.view(1, heads, frames, tpf, d), v.view(1, heads, frames, tpf, d)
        out = torch.empty_like(q)
        slots = np.arange(frames, dtype=np.int32)
        t_lf = med_ms(lambda: lf.lf_block_sparse_attn(g, q, kc, vc, slots, None, None, 1.0 / math.sqrt(d), out,
                                                      None, stream))
        row = {"heads": heads, "tokens": n, "head_dim": d, "flops": flops, "lf_us": round(t_lf * 1e3, 1),
               "lf_tflops": round(flops / (t_lf * 1e-3) / 1e12, 1)}
        for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
            try:
                with sdpa_kernel([be]):
                    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
                    t = med_ms(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v))
                row[f"sdpa_{name}_us"] = round(t * 1e3, 1)
                row[f"sdpa_{name}_tflops"] = round(flops / (t * 1e-3) / 1e12, 1)
                row[f"max_abs_diff_vs_sdpa_{name}"] = float((out.float() - ref.float()).abs().max().item())
            except RuntimeError as e:  # backend not built for this device
                row[f"sdpa_{name}"] = f"unavailable: {str(e)[:120]}"
        rows.append(row)
        del q, k, v, kc, vc, out
        torch.cuda.empty_cache()
    return rows


def cpu_baseline(w, x, k_frames, k_blocks, sample_qblocks: int):
    """The oracle, untuned, on the host cores: full compress + select, attention on a sample of query blocks."""
    from oracle import lf_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames)
    t1 = time.perf_counter()
    s = O.select(c["q_blk"], c["k_blk"], c["k_frm"], w.hist_frames, w.n_sink, w.blocks_per_frame, k_frames, k_blocks)
    t2 = time.perf_counter()
    rng = np.random.default_rng(0)
    all_q = [(b, h, qb) for b in range(w.batch) for h in range(w.heads) for qb in range(w.n_qblocks)]
    n_pick = len(all_q) if sample_qblocks <= 0 else min(sample_qblocks, len(all_q))
    pick = [all_q[i] for i in sorted(rng.choice(len(all_q), size=n_pick, replace=False))]
    scale = 1.0 / math.sqrt(w.head_dim)
    t3 = time.perf_counter()
    O.attention(x["q"], x["k_cache"], x["v_cache"], x["frame_slot"], s["sel_blocks"], s["n_sel"], w.tokens_per_frame,
                w.block, w.chunk_frames, w.hist_frames, scale, qblocks=pick)
    t4 = time.perf_counter()
    t_attn_full = (t4 - t3) * len(all_q) / len(pick)
    t_step = (t1 - t0) + (t2 - t1) + t_attn_full
    flops = effective_flops(w, s["sel_blocks"], s["n_sel"])
    return {
        "value": float(flops / t_step / 1e12), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"full oracle compress ({t1 - t0:.2f}s) + select ({t2 - t1:.2f}s) of one {w.name} call; "
                   f"float64 dense-masked attention on {len(pick)} of {len(all_q)} query blocks "
                   f"({t4 - t3:.2f}s), scaled to all of them; {t_step:.1f}s per call"),
        "s_per_step": t_step,
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Leg:
    """One workload on the GPU: seeded input sets resident in HBM, the step (host slot table and budget, then
    compress -> select -> attention, or fused selection -> attention), and its timing."""

    def __init__(self, w, n_sets: int, path: str):
        import torch

        from block_sparse_attention_lf_amd import inputs as I
        from block_sparse_attention_lf_amd import lf

        self.torch, self.lf, self.w, self.path = torch, lf, w, path
        self.g = lf.geom_of(w)
        self.scale = 1.0 / math.sqrt(w.head_dim)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        print(f"[bench] workload {w.name}: drawing {n_sets} input set(s)", file=sys.stderr, flush=True)
        self.sets, self.host0 = [], None
        for i in range(n_sets):
            x = I.make_inputs(w, seed=w.seed + 1000 * i)
            if i == 0:
                self.host0 = x
            self.sets.append(tuple(torch.from_numpy(x[k]).to(tdt).cuda() for k in ("q", "k_cache", "v_cache")))
            del x
        self.set_bytes = sum(t.numel() * t.element_size() for t in self.sets[0])
        self.bufs = lf.Buffers(self.g, w.k_frames, w.k_blocks)
        self.stream = torch.cuda.current_stream()
        self.slots = self.host_side()
        assert list(self.slots) == self.host0["frame_slot"].tolist()
        # effective FLOPs of each input set (selection is deterministic per set)
        self.flops = []
        for dev in self.sets:
            lf.hsa_attention(self.g, *dev, self.slots, self.bufs, self.scale)
            torch.cuda.synchronize()
            self.flops.append(effective_flops(w, self.bufs.sel_blocks.cpu().numpy(), self.bufs.n_sel.cpu().numpy()))
        self.pooled, self.commit_ms = [], None
        if path == "fused":
            self._pool_on_commit()

    def use_path(self, path: str):
        """Switch the steps to the other path on the same input sets (pooling on commit when first needed)."""
        self.path = path
        if path == "fused" and not self.pooled:
            self._pool_on_commit()

    def host_side(self):
        # a0: slot table of the cache for this chunk; a6: chunk budget (single call: its own sparsity)
        w, lf = self.w, self.lf
        hist, slots, _ = lf.lf_cache_frame_slots(w.policy, w.cache_slots, w.n_sink, w.chunk_frames, w.chunk_index)
        lf.lf_chunk_budget([1.0], None, [False], w.sparsity, w.sparsity, [hist], [w.n_sink], w.blocks_per_frame,
                           w.k_frames)
        return slots

    def _pool_on_commit(self):
        # the pooled keys of every history frame live in a slot-indexed cache,
        # filled when the frame is committed (once per frame, not per step)
        torch, lf, w, g = self.torch, self.lf, self.w, self.g
        S, nb, d = w.cache_slots, w.blocks_per_frame, w.head_dim
        hist_slots = [int(x) for x in self.slots[:w.hist_frames]]
        for q, kc, vc in self.sets:
            kp = (torch.empty((w.batch, w.heads, S, nb, d), dtype=torch.float32, device="cuda"),
                  torch.empty((w.batch, w.heads, S, d), dtype=torch.float32, device="cuda"))
            lf.lf_pool_keys(g, kc, hist_slots, kp[0], kp[1], self.stream)
            self.pooled.append(kp)
        # cost of one commit: pooling the chunk's own frames (they become history)
        chunk_slots = [int(x) for x in self.slots[w.hist_frames:w.hist_frames + w.chunk_frames]]
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        times = []
        n = len(self.sets)
        for r in range(6):
            kc = self.sets[r % n][1]
            cev[0].record(self.stream)
            lf.lf_pool_keys(g, kc, chunk_slots, self.pooled[r % n][0], self.pooled[r % n][1], self.stream)
            cev[1].record(self.stream)
            torch.cuda.synchronize()
            times.append(cev[0].elapsed_time(cev[1]))
        self.commit_ms = float(np.median(times[1:]))
        for (q, kc, vc), kp in zip(self.sets, self.pooled):  # restore the history pooling the steps read
            lf.lf_pool_keys(g, kc, hist_slots, kp[0], kp[1], self.stream)
        torch.cuda.synchronize()

    def step(self, i, ev=None, stage_ev=False):
        # ev: events around the attention launch (the roofline's kernel time);
        # stage_ev: two more around the first stage(s), for the stage split only
        # (each timing event costs the GPU a few microseconds per step, so the
        # timed steps carry just the two the roofline needs).
        lf, w, g, bufs, stream = self.lf, self.w, self.g, self.bufs, self.stream
        q, kc, vc = self.sets[i % len(self.sets)]
        sl = self.host_side()
        if stage_ev:
            ev[0].record(stream)
        if self.path == "fused":
            kp_blk, kp_frm = self.pooled[i % len(self.sets)]
            if stage_ev:
                ev[1].record(stream)
            lf.lf_select_fused(g, q, kp_blk, kp_frm, sl, w.k_frames, w.k_blocks, bufs.sel_frames, bufs.sel_blocks,
                               bufs.n_sel, None, stream)
        else:
            lf.lf_compress(g, q, kc, sl, bufs.q_blk, bufs.k_blk, bufs.k_frm, stream)
            if stage_ev:
                ev[1].record(stream)
            lf.lf_select(g, bufs.q_blk, bufs.k_blk, bufs.k_frm, w.k_frames, w.k_blocks, bufs.sel_frames,
                         bufs.sel_blocks, bufs.n_sel, stream)
        if ev is not None:
            ev[2].record(stream)
        lf.lf_block_sparse_attn(g, q, kc, vc, sl, bufs.sel_blocks, bufs.n_sel, self.scale, bufs.out, None, stream)
        if ev is not None:
            ev[3].record(stream)

    def time(self, steps: int, warmup: int) -> dict:
        """Exactly `steps` steps between two device synchronisations (after `warmup` untimed ones), HIP events
        around each attention launch; then a separate pass with events around every stage for the split."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        # The cyclic garbage collector is paused inside the timed region: a full
        # pass over a process holding torch takes tens of milliseconds and would
        # land in a random step.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            self.step(i, sevs[i], stage_ev=True)
        torch.cuda.synchronize()
        w = self.w
        ms_step = (t1 - t0) * 1e3 / steps
        attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        first_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sevs]))
        sel_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in sevs]))
        flops = float(np.mean([self.flops[i % len(self.sets)] for i in range(steps)]))
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        attn_tflops = flops / (attn_ms * 1e-3) / 1e12
        r = {"ms_per_step": ms_step, "attn_ms": attn_ms, "flops": flops, "attn_tflops": attn_tflops,
             "attn_frac": attn_tflops / peak, "peak": peak, "value": flops / (ms_step * 1e-3) / 1e12,
             "select_ms": sel_ms}
        if self.path == "fused":
            r["stages_ms"] = {"select_fused": sel_ms, "attention": attn_ms}
        else:
            cbytes = compress_bytes(w)
            gbs = cbytes / (first_ms * 1e-3) / 1e9
            r["stages_ms"] = {"compress": first_ms, "select": sel_ms, "attention": attn_ms}
            r["compress"] = {"bound": "hbm", "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS,
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": cbytes}
        return r


def path_comparison(leg: "Leg", r: dict, steps: int, warmup: int) -> dict:
    """The step path and the pool-on-commit path on the same input sets, one after the other in this process:
    ms per step and stage times of each (r: the timing already taken on the leg's current path)."""
    first = leg.path
    other = "fused" if first == "step" else "step"
    leg.use_path(other)
    ro = leg.time(steps, warmup)
    leg.use_path(first)
    res = {first: r, other: ro}
    out = {p: {"ms_per_step": round(x["ms_per_step"], 4), "stages_ms": {k: round(v, 4) for k, v in x["stages_ms"].items()}}
           for p, x in res.items()}
    out["fused"]["ms_per_commit"] = round(leg.commit_ms, 4)
    out["fused"]["frames_per_commit"] = leg.w.chunk_frames
    out["fused_over_step"] = round(res["fused"]["ms_per_step"] / res["step"]["ms_per_step"], 4)
    return out


def config_summary(leg: "Leg", r: dict, steps: int) -> dict:
    """Per-workload figures on the bench's own clock (the extra configurations)."""
    out = {"steps": steps, "input_sets_rotated": len(leg.sets), "ms_per_step": round(r["ms_per_step"], 4),
           "effective_gflop_per_step": round(r["flops"] / 1e9, 2),
           "step_tflops": round(r["value"], 1),
           "attention": {"avg_launch_ms": round(r["attn_ms"], 4), "achieved": round(r["attn_tflops"], 1),
                         "peak": r["peak"], "unit": "TFLOP/s", "frac": round(r["attn_frac"], 4)},
           "stages_ms": {k: round(v, 4) for k, v in r["stages_ms"].items()}}
    if "compress" in r:
        out["compress"] = r["compress"]
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); split over GPUs, the work would shard by head with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_attention_lf_amd import inputs as I
    from block_sparse_attention_lf_amd import lf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = I.WORKLOADS[args.workload] if args.workload else I.WAN480P_CHUNK
    leg = Leg(w, max(1, args.sets), args.path)
    g, scale, slots, bufs, stream = leg.g, leg.scale, leg.slots, leg.bufs, leg.stream
    host0 = leg.host0
    sets = leg.sets
    K = args.steps
    r = leg.time(K, args.warmup)
    ms_step, attn_ms, flops_mean, attn_tflops, peak = r["ms_per_step"], r["attn_ms"], r["flops"], r["attn_tflops"], \
        r["peak"]
    value = r["value"]
    traffic = traffic_from_profiles(w.name)

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1)/sqrt(d) q/k/v; no weights)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "tokens_per_frame": w.tokens_per_frame, "block": w.block, "chunk_frames": w.chunk_frames,
                   "hist_frames": w.hist_frames, "k_frames": w.k_frames, "k_blocks": w.k_blocks,
                   "sparsity": w.sparsity, "input_sets_rotated": len(leg.sets), "path": args.path,
                   "bytes_per_input_set": int(leg.set_bytes)},
        "roofline": {"bound": "mfma", "kernel": "attn_kernel (lf_block_sparse_attn)",
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": traffic,
                     "algorithmic_flops_per_launch": flops_mean, "avg_launch_ms": round(attn_ms, 4)},
        "stages_ms": {k: round(v, 4) for k, v in r["stages_ms"].items()},
        "attention_pct_of_mfma_peak": round(100 * attn_tflops / peak, 2),
    }
    if "compress" in r:
        result["compress"] = r["compress"]
    if args.path == "fused":
        result["pool_on_commit"] = {"ms_per_commit": round(leg.commit_ms, 4), "frames_per_commit": w.chunk_frames}
    if not args.headline_only:
        # the other path on the same inputs, after the timed region
        result["paths"] = path_comparison(leg, r, K, args.warmup)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 2
        src_t = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src_t)
        torch.cuda.synchronize()
        torch.neg(src_t, out=dst)  # reads and writes exactly n bf16 values
        torch.cuda.synchronize()
        result["calibration_copy_bytes_each_way"] = n * 2
    if args.backward and w.dtype == "bf16":
        # Backward of the same attention calls: out/lse from one forward per input set,
        # then `steps` timed backward launches (HIP events on the launch stream).
        # Algorithmic work: dV, dP, dQ and dK products, 8*d flops per visible
        # (query, key) pair = twice the forward's effective FLOPs.
        bw = []
        fb = lf.Buffers(g, w.k_frames, w.k_blocks, with_lse=True)
        for i, (q, kc, vc) in enumerate(sets):
            lf.hsa_attention(g, q, kc, vc, slots, fb, scale)
            o = fb.out.clone()
            ls = fb.lse.clone()
            gen = torch.Generator(device="cuda").manual_seed(100 + i)
            do = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            bw.append((o, ls, do, fb.sel_blocks.clone(), fb.n_sel.clone()))
        delta = torch.empty(sets[0][0].shape[:3], dtype=torch.float32, device="cuda")
        dq = torch.empty(sets[0][0].shape, dtype=torch.float32, device="cuda")
        dk = torch.empty(sets[0][1].shape, dtype=torch.float32, device="cuda")
        dv = torch.empty(sets[0][1].shape, dtype=torch.float32, device="cuda")

        def bwd(i):
            q, kc, vc = sets[i % len(sets)]
            o, ls, do, sb, nsl = bw[i % len(sets)]
            lf.lf_block_sparse_attn_bwd(g, q, kc, vc, slots, sb, nsl, scale, o, ls, do, delta, dq, dk, dv, stream)

        for i in range(args.warmup):
            bwd(i)
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            bev[i][0].record(stream)
            bwd(i)
            bev[i][1].record(stream)
        torch.cuda.synchronize()
        bms = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
        bflops = 2.0 * flops_mean
        result["backward"] = {"ms_per_call": round(bms, 4), "algorithmic_flops": bflops,
                              "achieved": round(bflops / (bms * 1e-3) / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                              "frac": round(bflops / (bms * 1e-3) / 1e12 / peak, 4),
                              "kernels": "bwd_dq_kernel + bwd_dkv_kernel (current-chunk and history dK+dV passes)"}
    if args.fp8 and w.dtype == "bf16" and w.head_dim == 128:
        # The same attention calls with queries and keys as MX-FP8 (E4M3 codes,
        # one E8M0 scale per 32 channels, quantised on the host, untimed) and
        # the bf16 step's selections. Score products run at the FP8 MFMA rate
        # and PV products at the bf16 one: with equal FLOPs in each, the
        # kernel's roofline is 1 / (0.5/P_fp8 + 0.5/P_bf16).
        print("[bench] quantising the input sets to MX-FP8", file=sys.stderr, flush=True)
        f8 = []
        for i, (q, kc, vc) in enumerate(sets):
            lf.hsa_attention(g, q, kc, vc, slots, bufs, scale)
            q8, qs = I.mx_quantize(q.float().cpu().numpy())
            k8, ks = I.mx_quantize(kc.float().cpu().numpy())
            f8.append(tuple(torch.from_numpy(a).cuda() for a in (q8, qs, k8, ks)) +
                      (bufs.sel_blocks.clone(), bufs.n_sel.clone()))
        out8 = torch.empty_like(bufs.out)

        def fwd8(i):
            q8, qs, k8, ks, sb, nsl = f8[i % len(sets)]
            lf.lf_block_sparse_attn_fp8(g, q8, qs, k8, ks, sets[i % len(sets)][2], slots, sb, nsl, scale, out8, None,
                                        stream)

        for i in range(args.warmup):
            fwd8(i)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            fev[i][0].record(stream)
            fwd8(i)
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        fms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
        fpeak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        fach = flops_mean / (fms * 1e-3) / 1e12
        result["fp8"] = {"ms_per_call": round(fms, 4), "algorithmic_flops": flops_mean, "achieved": round(fach, 2),
                         "peak": round(fpeak, 1), "unit": "TFLOP/s", "frac": round(fach / fpeak, 4),
                         "frac_of_bf16_peak": round(fach / PEAK_BF16_TFLOPS, 4),
                         "speedup_vs_bf16_attention": round(attn_ms / fms, 3),
                         "kernel": "attn_kernel Q8 (lf_block_sparse_attn_fp8)"}
    if args.dense_vs_sdpa:
        print("[bench] dense attention against torch SDPA", file=sys.stderr, flush=True)
        result["dense_vs_sdpa"] = dense_vs_sdpa(max(args.warmup, 2), max(K, 5))
    if not args.headline_only:
        # The other workloads on the same clock: long history with a sink and the
        # wide-head case (one input set each beyond what the MALL holds), then
        # the chunk-wise rollout. Each leg frees its inputs before the next.
        del leg, sets, bufs
        torch.cuda.empty_cache()
        extra = {}
        for wl, n_sets, steps in ((I.LONG_HISTORY_SINK, 2, 10), (I.WIDE_HEAD, 1, 5)):
            if wl.name == w.name:
                continue
            lg = Leg(wl, n_sets, args.path)
            rr = lg.time(steps, 2)
            extra[wl.name] = config_summary(lg, rr, steps)
            extra[wl.name]["paths"] = path_comparison(lg, rr, steps, 2)
            del lg
            torch.cuda.empty_cache()
        result["configs"] = extra
        print("[bench] chunk rollout", file=sys.stderr, flush=True)
        result["rollout"] = rollout(max(args.warmup, 1))
    if args.cpu_single_thread:
        # The oracle with BLAS held to one thread: the tiny fp32 case whole, and
        # the 480p chunk call (compress + select + attention on 150 sampled
        # query blocks, scaled to all 900).
        from threadpoolctl import threadpool_limits

        st = {}
        with threadpool_limits(limits=1):
            for wl, sample in ((I.TINY_FP32, 0), (I.WAN480P_CHUNK, 150)):
                xs = I.make_inputs(wl)
                rr = cpu_baseline(wl, xs, wl.k_frames, wl.k_blocks, sample)
                st[wl.name] = {"s_per_call": round(rr["s_per_step"], 4), "sample": rr["sample"]}
        result["cpu_single_thread"] = st
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, host0, w.k_frames, w.k_blocks, args.cpu_sample_qblocks)
        cb.pop("s_per_step")
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
