"""A seeded sweep of small random shapes through the whole path, against the
fp64 oracle: phase 1, then the query step and every decode step, each as one
star_attn_decode_step call and again as separate calls (append, partials,
merge), and on a paged cache, whose results must be the contiguous cache's
bits; and phase 1 with the rotary embedding in both anchor position-id modes. The shapes mix batch, GQA ratio (1 to 8), head dimension, contexts
from one token up, blocks from one row to longer than the context, anchors
shorter than the block and off the 32-key grid, and query steps from one
token to a wide tile, in bf16 and fp32. They come from a fixed seed, so the
sweep is the same every run; each case prints its shape before it runs."""
import numpy as np
import pytest
import torch

import long_context_attention_phase1_amd as sa
from long_context_attention_phase1_amd import synthetic as syn
from long_context_attention_phase1_amd.pipeline import PagedPipeline, Pipeline, to_host_f64
from oracle import star_oracle as orc

pytestmark = pytest.mark.gpu

# the bars of the parity tests (tests/test_gpu_parity.py derives them)
TOL = {"bf16": 2e-2, "f32": 1e-5}
TOL_LSE = {"bf16": 4e-3, "f32": 1e-5}


def _shapes(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 3 == 2 else "bf16"
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        L = int(rng.choice([1, int(rng.integers(2, 100)), int(rng.integers(100, 600))],
                           p=[0.1, 0.3, 0.6]))
        b = int(rng.choice([1, int(rng.integers(1, L + 1)), 64 * int(rng.integers(1, 6)),
                            L + int(rng.integers(0, 50))]))
        b = max(1, b)
        a = int(rng.integers(1, b + 1))
        Tq = int(rng.choice([1, int(rng.integers(2, 9)), int(rng.integers(9, 48))]))
        Td = int(rng.integers(1, 4))
        out.append(syn.Workload(f"rand{i}", B, G * Hkv, Hkv, d, L, b, a, Tq, Td, dtype,
                                seed=100 + i))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_random_shape_matches_oracle(w):
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    print(f"{w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
          f"L={w.ctx_len} b={w.block_len} a={w.anchor_len} Tq={w.n_query} Td={w.n_decode} "
          f"{w.dtype}", flush=True)
    p = Pipeline(w, threads=4)
    p.write_context()
    o1 = to_host_f64(p.phase1())
    fused_o, fused_l = p.run_tail(fused=True)
    torch.cuda.synchronize()

    q = Pipeline(w, inputs=p.inputs, threads=4)
    q.write_context()
    sep_o, sep_l = q.run_tail(fused=False)
    # the paged cache (a random page permutation) gives the contiguous cache's bits
    r = PagedPipeline(w, inputs=p.inputs, threads=4)
    r.write_context()
    pg_o, pg_l = r.run_tail(fused=True)
    torch.cuda.synchronize()
    assert np.array_equal(pg_o, fused_o) and np.array_equal(pg_l, fused_l), w.name

    x = {k: syn.to_f64(v, w.dtype) for k, v in p.inputs.items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    ref1 = orc.phase1(x["q_ctx"], x["k_ctx"], x["v_ctx"], w.block_len, w.anchor_len, sc)
    ref_o, ref_l = orc.decode_loop(x["q_tail"], x["k_ctx"], x["v_ctx"], x["k_tail"],
                                   x["v_tail"], w.n_query, sc)
    e1 = float(np.max(np.abs(o1 - ref1)))
    errs = [(float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(l - ref_l))))
            for o, l in ((fused_o, fused_l), (sep_o, sep_l))]
    print(f"{w.name}: phase 1 {e1:.2e}; tail (fused) o {errs[0][0]:.2e} lse {errs[0][1]:.2e}; "
          f"(separate) o {errs[1][0]:.2e} lse {errs[1][1]:.2e}")
    assert np.isfinite(o1).all() and e1 <= TOL[w.dtype]
    for eo, el in errs:
        assert eo <= TOL[w.dtype] and el <= TOL_LSE[w.dtype]

    # phase 1 with the rotary embedding fused in, both anchor position-id modes
    for mode, omode, mname in ((sa.STAR_ROPE_ORIGINAL, orc.ROPE_ORIGINAL, "original"),
                               (sa.STAR_ROPE_ADJACENT, orc.ROPE_ADJACENT, "adjacent")):
        rope = p.rope(mode)
        p.write_context_rope(rope)
        o = to_host_f64(p.phase1_rope(rope))
        torch.cuda.synchronize()
        c, sn = (t.astype(np.float64) for t in p.rope_host)
        ref = orc.phase1_rope(x["q_ctx"], x["k_ctx"], x["v_ctx"], w.block_len, w.anchor_len, sc,
                              c, sn, omode)
        er = float(np.max(np.abs(o - ref)))
        print(f"{w.name}: phase 1 with rotary ids ({mname}) {er:.2e}")
        assert er <= TOL[w.dtype], (w.name, mname)
