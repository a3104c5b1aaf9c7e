"""Writes the golden fixtures in this folder from the CPU oracle only.

Run from the repository root:  python tests/golden/make_golden.py
Inputs come from the seeded generators; every stored value is an oracle
output. Citations: Light Forcing technical summary 2.2 (selection) and 2.1
(chunk-aware growth); press summary section 1 (seven chunks, first dense).
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from block_sparse_attention_lf_amd import inputs as I  # noqa: E402
from oracle import lf_oracle as O  # noqa: E402


def tiny_selection():
    w = I.TINY_FP32
    x = I.make_inputs(w)
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames)
    s = O.select(c["q_blk"], c["k_blk"], c["k_frm"], w.hist_frames, w.n_sink, w.blocks_per_frame, w.k_frames, w.k_blocks)
    return {
        "citation": "Light Forcing, technical summary 2.2: frame top-k then block top-k inside chosen frames",
        "workload": w.name,
        "frame_slot": x["frame_slot"].tolist(),
        "sel_frames": s["sel_frames"].tolist(),
        "sel_blocks": s["sel_blocks"].tolist(),
        "n_sel": s["n_sel"].tolist(),
    }


def rollout_budget():
    r = I.CHUNK_ROLLOUT
    n = r.n_chunks
    out = O.chunk_budget(r.sigmas(), [1.0] * n, [True] + [False] * (n - 1), r.s_base, r.s_target,
                         [r.chunk_frames * i for i in range(n)], [0] * n, r.blocks_per_frame, r.k_frames_min)
    return {
        "citation": "Light Forcing, technical summary 2.1: s_i = s_base - alpha_i beta, alpha_i = 1/sqrt(sigma_i); "
                    "press summary section 1: seven chunks, first chunk dense",
        "rollout": r.name, "sigma": r.sigmas(), "s_base": r.s_base, "s_target": r.s_target,
        "beta": out["beta"], "sparsity": out["sparsity"],
        "k_frames": out["k_frames"], "k_blocks": out["k_blocks"],
    }


if __name__ == "__main__":
    for name, fn in (("tiny_fp32_selection.json", tiny_selection), ("chunk_rollout_budget.json", rollout_budget)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
            f.write("\n")
        print("wrote", name)
