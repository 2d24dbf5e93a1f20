"""Writes tests/golden/tiny_ragged_bf16.json from the fp64 oracle only.

Run from the repository root: ``python -m tests.golden.make_golden``.
The workload is a small bf16 case with a ragged last block, an anchor shorter
than the block, GQA 2:1 and a three-token causal tail; its inputs come from
the seeded generator, its expected values from ``oracle/`` alone.
"""
import json
import os

from long_context_attention_phase1_amd import synthetic as syn
from oracle import star_oracle as orc

W = syn.Workload("tiny_ragged_bf16", 1, 2, 1, 64, 40, 16, 10, 3, 0, "bf16", seed=7)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_ragged_bf16.json")


def expected():
    x = syn.make_inputs(W, threads=1)
    f = {k: syn.to_f64(v, W.dtype) for k, v in x.items()}
    sc = orc.resolve_scale(W.head_dim, 0.0)
    o1 = orc.phase1(f["q_ctx"], f["k_ctx"], f["v_ctx"], W.block_len, W.anchor_len, sc)
    import numpy as np
    k_all = np.concatenate([f["k_ctx"], f["k_tail"]], axis=1)
    v_all = np.concatenate([f["v_ctx"], f["v_tail"]], axis=1)
    pos = [W.ctx_len + j for j in range(W.n_query)]
    o2, l2 = orc.phase2_dense(f["q_tail"], k_all, v_all, pos, sc)
    return o1, o2, l2


def main():
    o1, o2, l2 = expected()
    doc = {
        "about": "Expected fp64 oracle outputs for a small Star Attention case "
                 "(ragged last block, anchor shorter than the block, GQA 2:1). "
                 "Written by tests/golden/make_golden.py, which calls only oracle/.",
        "workload": {k: getattr(W, k) for k in ("name", "batch", "n_q_heads", "n_kv_heads",
                                                "head_dim", "ctx_len", "block_len", "anchor_len",
                                                "n_query", "n_decode", "dtype", "seed")},
        "phase1_out": [float(f"{x:.17g}") for x in o1.ravel()],
        "phase2_out": [float(f"{x:.17g}") for x in o2.ravel()],
        "phase2_lse": [float(f"{x:.17g}") for x in l2.ravel()],
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))


if __name__ == "__main__":
    main()
