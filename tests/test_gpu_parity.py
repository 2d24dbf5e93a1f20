"""GPU parity: libstarattn (through the C ABI) against the fp64 oracle.

Small workloads checked element by element: several tiles, ragged last
blocks, block starts not aligned to the 64-row cache tile, anchors shorter
than the block, one-row blocks and a one-token context, GQA 1:1 / 2:1 / 4:1 / 8:1, head_dim 64 and 128, bf16 and
fp32, the peaked-softmax input, a context shorter than one block, both
phase-2 kernels (<= 32 and > 32 query columns), empty splits and every
decode step. Tolerances: max-abs 1e-5 (fp32 workloads) and 2e-2 (bf16
outputs, fp32 accumulation).
"""
import json
import os

import numpy as np
import pytest
import torch

import long_context_attention_phase1_amd as sa
from long_context_attention_phase1_amd import synthetic as syn
from oracle import star_oracle as orc
from long_context_attention_phase1_amd.pipeline import Pipeline, to_host_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
# the kernels sum the bf16-rounded P (the same weights that P.V uses): each
# term is off by at most 2^-8 relative (8 significant bits, round to
# nearest), so the sum is too, and the lse by at most -ln(1 - 2^-8) = 3.92e-3,
# a bound that a row dominated by one key can approach
TOL_LSE = {"bf16": 4e-3, "f32": 1e-5}

W = syn.Workload
CASES = {
    "tiny_f32": syn.WORKLOADS["tiny_f32"],
    "gqa4_d128_ragged": W("gqa4_d128_ragged", 1, 8, 2, 128, 640, 256, 256, 8, 3, "bf16", seed=1),
    "g1_unaligned_a_lt_b": W("g1_unaligned", 2, 4, 4, 128, 333, 100, 37, 5, 2, "bf16", seed=2),
    "g2_d64_wide_tail": W("g2_d64", 1, 4, 2, 64, 300, 128, 64, 20, 2, "bf16", seed=3),
    "g8_narrow": W("g8", 1, 16, 2, 128, 256, 64, 64, 4, 2, "bf16", seed=4),
    "peaked": W("peaked", 1, 4, 1, 128, 512, 128, 128, 3, 2, "bf16", peak_frac=0.05,
                peak_factor=8.0, seed=5),
    "one_block": W("one_block", 1, 4, 1, 128, 200, 256, 100, 2, 1, "bf16", seed=6),
    "f32_gqa_d128": W("f32_gqa", 1, 4, 2, 128, 130, 64, 10, 3, 2, "f32", seed=7),
    "g4_d64_many_blocks": W("g4_d64", 1, 8, 2, 64, 1024, 128, 128, 40, 1, "bf16", seed=8),
    # tail longer than one split: early query rows see nothing of the second tail split
    "long_tail_wide": W("long_tail", 1, 4, 2, 128, 128, 64, 64, 300, 1, "bf16", seed=13),
    # balanced decode plan on a ragged context: the tail start (2172) falls
    # inside a 32-key slice of the range [2048, 2176), and the last range
    # [2176, 2180) holds query rows only, so the first four queries see none
    # of it (an empty split: lse = -inf, o = 0)
    "ragged_empty_split": W("ragged_empty", 1, 4, 1, 128, 2172, 1024, 300, 8, 2, "bf16", seed=14),
    # balanced decode plan: 512-row ranges with a block start (1088) and the
    # tail start (2176) strictly inside, a 16-column query step, tail < 1 tile
    "balanced_bnd": W("balanced_bnd", 1, 8, 2, 128, 2176, 1088, 512, 4, 3, "bf16", seed=15),
    # per-wave decode kernel at d = 64, two sequences, GQA 8:1, a 24-column
    # query step; block starts 448 and 1344 fall inside 128-row ranges
    "balanced_b2_g8_d64": W("bal_b2", 2, 16, 2, 64, 1536, 448, 200, 3, 2, "bf16", seed=16),
    # degenerate partitions: one-row blocks and a one-row anchor (every row
    # sees token 0 and itself), a one-token context, one-row blocks with a
    # query step of more than 32 columns, and the fp32 path
    "b1_a1": W("b1_a1", 1, 4, 2, 128, 70, 1, 1, 3, 2, "bf16", seed=17),
    "ctx1": W("ctx1", 1, 2, 1, 64, 1, 1, 1, 2, 2, "bf16", seed=18),
    "b1_wide_tail": W("b1_wide", 1, 4, 2, 128, 50, 1, 1, 40, 2, "bf16", seed=20),
    "f32_b1": W("f32_b1", 1, 2, 2, 64, 40, 1, 1, 2, 1, "f32", seed=19),
    # eight kv groups (2 sequences x 4 kv heads), GQA 8:1 in two head
    # sub-groups, a 320-column query step: both sub-groups read each split,
    # so the wide kernel keeps a kv head's work items on one XCD and reads
    # K/V with the default cache policy
    "kv_major_g8": W("kv_major", 2, 32, 4, 128, 640, 256, 256, 40, 1, "bf16", seed=21),
    # query steps of 1,024 or more (query, head) rows: the merge takes one
    # wave per row (d = 128 and 64, bf16 and fp32)
    "many_rows_d64": W("many_rows_d64", 1, 16, 4, 64, 700, 256, 128, 70, 1, "bf16", seed=22),
    "f32_many_rows": W("f32_many_rows", 1, 8, 2, 64, 200, 64, 32, 130, 1, "f32", seed=23),
    # a query step of at most half a query tile with four heads per workgroup
    # (as the 1M workload's 32 query rows): the waves holding rows 32..63 only
    # load tiles and meet barriers, and their SIMD partners do the arithmetic
    "short_tile_g4": W("short_tile_g4", 1, 8, 2, 128, 2100, 512, 300, 24, 2, "bf16", seed=24),
    # fp32 on two sequences: ragged last block, anchor shorter than the block
    # and off the 32-key grid, so a workgroup's slices mix anchor and block
    # keys and its four waves take different numbers of them
    "f32_b2_ragged": W("f32_b2_ragged", 2, 4, 2, 64, 333, 100, 37, 5, 2, "f32", seed=25),
}
EMPTY_SPLIT_CASES = ("long_tail_wide", "ragged_empty_split")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")


def _f64(w, x):
    return syn.to_f64(x, w.dtype)


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


@pytest.fixture(scope="module")
def runs():
    _need_gpu()
    return {}


def _pipeline(runs, name):
    if name not in runs:
        w = CASES[name]
        p = Pipeline(w, threads=4)
        p.write_context()
        o1 = to_host_f64(p.phase1())
        tail_o, tail_l = p.run_tail()
        torch.cuda.synchronize()
        runs[name] = (p, o1, tail_o, tail_l)
    return runs[name]


@pytest.mark.parametrize("name", list(CASES))
def test_phase1_matches_oracle(runs, name):
    p, o1, _, _ = _pipeline(runs, name)
    w = p.w
    x = {k: _f64(w, v) for k, v in p.inputs.items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    ref = orc.phase1(x["q_ctx"], x["k_ctx"], x["v_ctx"], w.block_len, w.anchor_len, sc)
    assert np.isfinite(o1).all()
    err = _err(o1, ref)
    print(f"{name}: phase-1 max-abs error {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name", list(CASES))
def test_phase2_query_and_decode_match_oracle(runs, name):
    p, _, tail_o, tail_l = _pipeline(runs, name)
    w = p.w
    x = {k: _f64(w, v) for k, v in p.inputs.items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    ref_o, ref_l = orc.decode_loop(x["q_tail"], x["k_ctx"], x["v_ctx"], x["k_tail"],
                                   x["v_tail"], w.n_query, sc)
    eo, el = _err(tail_o, ref_o), _err(tail_l, ref_l)
    print(f"{name}: phase-2 max-abs error o {eo:.3e}, lse {el:.3e}")
    assert eo <= TOL[w.dtype]
    assert el <= TOL_LSE[w.dtype]


@pytest.mark.parametrize("name", ["gqa4_d128_ragged", "g1_unaligned_a_lt_b", "g2_d64_wide_tail",
                                  "g8_narrow", "f32_gqa_d128", "long_tail_wide",
                                  "ragged_empty_split", "balanced_bnd", "balanced_b2_g8_d64",
                                  "b1_a1", "ctx1", "b1_wide_tail", "f32_b1", "short_tile_g4",
                                  "f32_b2_ragged"])
def test_partials_are_the_hosts_replies(runs, name):
    """Each split's (vector, scalar) equals the oracle's host reply on that range."""
    p, _, _, _ = _pipeline(runs, name)
    w = p.w
    x = {k: _f64(w, v) for k, v in p.inputs.items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    kv_len = w.ctx_len + w.n_query
    n_split, o_part, lse_part, _, _ = p.workspace(kv_len, w.n_query)
    sa.star_attn_phase2_partial(p.desc, p.k_cache, p.v_cache, kv_len, p.q_query, w.n_query,
                                o_part, lse_part)
    torch.cuda.synchronize()
    op, lp = o_part.cpu().numpy(), lse_part.cpu().numpy()
    k_all = np.concatenate([x["k_ctx"], x["k_tail"][:, :w.n_query]], axis=1)
    v_all = np.concatenate([x["v_ctx"], x["v_tail"][:, :w.n_query]], axis=1)
    G = w.group
    n_empty = 0
    for sg in range(n_split):
        lo, hi, host = sa.star_attn_phase2_split_range(p.desc, kv_len, w.n_query, sg)
        for s in range(w.batch):
            for j in range(w.n_query):
                for h in range(w.n_q_heads):
                    ro, rl = orc.phase2_partial(x["q_tail"][s, j, h], k_all[s, :, h // G],
                                                v_all[s, :, h // G], w.ctx_len + j, lo, hi, sc)
                    if rl == -np.inf:
                        n_empty += 1
                        assert lp[s, j, h, sg] == -np.inf and np.all(op[s, j, h, sg] == 0.0)
                        continue
                    tol = 1e-5 if w.dtype == "f32" else 1e-2
                    assert _err(op[s, j, h, sg], ro) <= tol, (sg, s, j, h)
                    assert abs(lp[s, j, h, sg] - rl) <= TOL_LSE[w.dtype]
    if name in EMPTY_SPLIT_CASES:
        assert n_empty > 0


def test_golden_fixture_on_gpu():
    _need_gpu()
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_ragged_bf16.json")
    doc = json.load(open(path))
    w = W(**doc["workload"])
    p = Pipeline(w, threads=1)
    p.write_context()
    o1 = to_host_f64(p.phase1()).ravel()
    o2, l2 = p.query_step()
    torch.cuda.synchronize()
    assert _err(o1, doc["phase1_out"]) <= TOL["bf16"]
    assert _err(to_host_f64(o2).ravel(), doc["phase2_out"]) <= TOL["bf16"]
    assert _err(l2.cpu().numpy().ravel(), doc["phase2_lse"]) <= TOL_LSE["bf16"]


def test_kv_write_layout_bit_exact():
    _need_gpu()
    for dtype, d in (("bf16", 128), ("bf16", 64), ("f32", 64)):
        w = W("layout", 2, 6, 3, d, 150, 64, 64, 9, 0, dtype, seed=9)
        p = Pipeline(w, threads=1)
        p.write_context()
        # tail rows in two unaligned pieces
        sa.star_kv_write(p.desc, p.k_cache, p.v_cache, w.ctx_len, p.k_query[:, :4].contiguous(),
                         p.v_query[:, :4].contiguous(), 4)
        sa.star_kv_write(p.desc, p.k_cache, p.v_cache, w.ctx_len + 5,
                         p.k_query[:, 5:9].contiguous(), p.v_query[:, 5:9].contiguous(), 4)
        torch.cuda.synchronize()
        R = -(-(w.ctx_len + w.tail_cap) // 64) * 64
        raw = np.uint16 if dtype == "bf16" else np.uint32
        kc = p.k_cache.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy().view(raw)
        vc = p.v_cache.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy().view(raw)
        kc = kc.reshape(w.batch, w.n_kv_heads, R, d)
        vc = vc.reshape(w.batch, w.n_kv_heads, R // 64, d, 64)
        k_rows = np.concatenate([p.inputs["k_ctx"], p.inputs["k_tail"][:, :9]], axis=1).view(raw)
        v_rows = np.concatenate([p.inputs["v_ctx"], p.inputs["v_tail"][:, :9]], axis=1).view(raw)
        nan = 0x7FC0 if dtype == "bf16" else np.float32(np.nan).view(np.uint32)
        for r in range(R):
            written = r < w.ctx_len + 4 or (w.ctx_len + 5 <= r < w.ctx_len + 9)
            for s in range(w.batch):
                for g in range(w.n_kv_heads):
                    kr = kc[s, g, r]
                    vr = vc[s, g, r // 64, :, r % 64]
                    if written:
                        assert np.array_equal(kr, k_rows[s, r, g]), (dtype, d, r, s, g)
                        assert np.array_equal(vr, v_rows[s, r, g]), (dtype, d, r, s, g)
                    else:
                        assert np.all(kr == nan) and np.all(vr == nan), (dtype, d, r)


def test_phase1_is_deterministic_and_blocks_independent():
    _need_gpu()
    w = W("indep", 1, 8, 2, 128, 768, 256, 256, 1, 0, "bf16", seed=10)
    p = Pipeline(w, threads=1)
    p.write_context()
    a = p.phase1().clone()
    b = p.phase1().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # perturb block 1 (rows 256..511): blocks 0 and 2 must not change at all
    p.dev["q_ctx"][:, 256:512] *= -1
    k2 = p.dev["k_ctx"].clone()
    v2 = p.dev["v_ctx"].clone()
    k2[:, 256:512] += 1.0
    v2[:, 256:512] -= 0.5
    sa.star_kv_write(p.desc, p.k_cache, p.v_cache, 0, k2, v2, w.ctx_len)
    c = p.phase1().clone()
    torch.cuda.synchronize()
    ai, ci = a.view(torch.int16), c.view(torch.int16)
    assert torch.equal(ai[:, :256], ci[:, :256])
    assert torch.equal(ai[:, 512:], ci[:, 512:])
    assert not torch.equal(ai[:, 256:512], ci[:, 256:512])


def test_phase2_is_deterministic():
    _need_gpu()
    w = CASES["gqa4_d128_ragged"]
    p = Pipeline(w, threads=1)
    p.write_context()
    o1, l1 = p.query_step()
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = p.query_step()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("d,n_query,n_split", [(128, 80, 7), (64, 70, 40), (128, 20, 5)])
def test_lse_merge_direct_against_oracle(d, n_query, n_split):
    """star_attn_lse_merge on crafted partials: random vectors and lse values,
    empty splits (lse = -inf) scattered, one row with no visible key at all.
    The first two shapes have 1,024 or more rows (one wave per row), the last
    fewer (one workgroup per row)."""
    _need_gpu()
    Hq = 16
    desc = sa.make_desc(1, Hq, 4, d, 64, 64, 64, n_query, sa.STAR_F32)
    rng = np.random.default_rng(d + n_query)
    rows = n_query * Hq
    o_part = rng.standard_normal((rows, n_split, d)).astype(np.float32)
    lse = (rng.standard_normal((rows, n_split)) * 3.0).astype(np.float32)
    lse[rng.random((rows, n_split)) < 0.2] = -np.inf
    o_part[np.isinf(lse)] = 0.0  # an empty split's vector is zero, as the kernels write it
    lse[5] = -np.inf
    o_part[5] = 0.0
    dev = lambda x: torch.from_numpy(x).cuda()
    op = dev(o_part).view(1, n_query, Hq, n_split, d)
    lp = dev(lse).view(1, n_query, Hq, n_split)
    o = torch.empty(1, n_query, Hq, d, dtype=torch.float32, device="cuda")
    ob = torch.empty(1, n_query, Hq, d, dtype=torch.bfloat16, device="cuda")
    l_out = torch.empty(1, n_query, Hq, dtype=torch.float32, device="cuda")
    sa.star_attn_lse_merge(desc, n_query, n_split, op, lp, o, sa.STAR_F32, l_out)
    sa.star_attn_lse_merge(desc, n_query, n_split, op, lp, ob, sa.STAR_BF16, None)
    torch.cuda.synchronize()
    got = o.cpu().numpy().reshape(rows, d).astype(np.float64)
    gotb = ob.float().cpu().numpy().reshape(rows, d).astype(np.float64)
    gl = l_out.cpu().numpy().reshape(rows).astype(np.float64)
    eo = el = eb = 0.0
    for r in range(rows):
        ro, rl = orc.lse_merge(o_part[r].astype(np.float64), lse[r])
        eo = max(eo, float(np.abs(got[r] - ro).max()))
        eb = max(eb, float(np.abs(gotb[r] - ro).max()))
        if np.isinf(rl):
            assert gl[r] == -np.inf and not got[r].any()
        else:
            el = max(el, abs(gl[r] - rl))
    assert eo <= 1e-5 and el <= 1e-5 and eb <= 2e-2, (eo, el, eb)


def test_binding_rejects_wrong_buffers():
    _need_gpu()
    w = CASES["g8_narrow"]
    p = Pipeline(w, threads=1)
    bad = torch.empty(1, 3, dtype=p.elt, device="cuda")
    with pytest.raises(ValueError):
        sa.star_attn_phase1(p.desc, p.k_cache, p.v_cache, bad, p.o_ctx)
    with pytest.raises(ValueError):
        sa.star_attn_phase1(p.desc, p.k_cache[:10], p.v_cache, p.dev["q_ctx"], p.o_ctx)
    with pytest.raises(sa.StarAttnError):
        sa.star_attn_phase2_plan(p.desc, w.ctx_len, 1)


@pytest.mark.parametrize("name", ["gqa4_d128_ragged", "g8_narrow", "peaked", "ragged_empty_split",
                                  "g1_unaligned_a_lt_b", "tiny_f32", "g4_d64_many_blocks",
                                  "balanced_bnd", "balanced_b2_g8_d64", "b1_a1", "ctx1",
                                  "f32_b1", "b1_wide_tail", "g2_d64_wide_tail", "long_tail_wide",
                                  "kv_major_g8", "many_rows_d64", "short_tile_g4", "f32_b2_ragged"])
def test_fused_decode_step(runs, name):
    """star_attn_decode_step (append + partials + merge) against the oracle's
    decode loop and against the three separate calls, every step: the query
    step (n_query rows in one call) and every decode step. The wide shapes
    (more than 32 columns) cover one and several query tiles and head
    sub-groups."""
    p0, _, tail_o, tail_l = _pipeline(runs, name)
    w = p0.w
    p = Pipeline(w, inputs=p0.inputs, threads=4)
    p.write_context()
    fo, fl = p.run_tail(fused=True)
    torch.cuda.synchronize()
    x = {k: _f64(w, v) for k, v in p.inputs.items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    ref_o, ref_l = orc.decode_loop(x["q_tail"], x["k_ctx"], x["v_ctx"], x["k_tail"],
                                   x["v_tail"], w.n_query, sc)
    d = slice(0, None)
    eo, el = _err(fo[:, d], ref_o[:, d]), _err(fl[:, d], ref_l[:, d])
    print(f"{name}: fused query and decode steps max-abs error o {eo:.3e}, lse {el:.3e}")
    assert eo <= TOL[w.dtype] and el <= TOL_LSE[w.dtype]
    # same partial arithmetic as the separate calls: outputs agree to the
    # output rounding (bf16: one ulp of |o| < 8 is 2^-5 at most)
    assert _err(fo[:, d], tail_o[:, d]) <= (1e-6 if w.dtype == "f32" else 2 ** -5)
    assert _err(fl[:, d], tail_l[:, d]) <= 1e-4
    # the appended rows landed in the cache exactly as star_kv_write puts them
    assert torch.equal(p.k_cache.view(torch.int16), p0.k_cache.view(torch.int16))
    assert torch.equal(p.v_cache.view(torch.int16), p0.v_cache.view(torch.int16))
