"""GPU parity of the rotary embedding fused into phase 1 (both anchor
position-id modes) and into the cache write, against the fp64 oracle.

The oracle rotates every query and key exactly at its position id (anchor
rows per mode) and attends; the kernels rotate K once at its cache row
(rounded to the cache dtype) and the query at its row, turned back by
i*b - a for the anchor pass of block i in the adjacent mode. Tolerances as
for phase 1: max-abs 2e-2 (bf16) and 1e-5 (fp32). The cache write is
checked bit for bit against the oracle's float32-then-bf16 rotation.
"""
import numpy as np
import pytest
import torch

import long_context_attention_phase1_amd as sa
from long_context_attention_phase1_amd import synthetic as syn
from oracle import star_oracle as orc
from long_context_attention_phase1_amd.pipeline import Pipeline, to_host_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
W = syn.Workload
MODES = {"original": sa.STAR_ROPE_ORIGINAL, "adjacent": sa.STAR_ROPE_ADJACENT}
ORC_MODE = {sa.STAR_ROPE_ORIGINAL: orc.ROPE_ORIGINAL, sa.STAR_ROPE_ADJACENT: orc.ROPE_ADJACENT}
CASES = {
    # several blocks, anchor = block (adjacent ids coincide with the original
    # ones for block 1 only), GQA 4:1
    "gqa4_d128_ragged": W("gqa4_d128_ragged", 1, 8, 2, 128, 640, 256, 256, 8, 3, "bf16", seed=1),
    # anchor shorter than the block, unaligned blocks and anchor edge tile
    "g1_unaligned_a_lt_b": W("g1_unaligned", 2, 4, 4, 128, 333, 100, 37, 5, 2, "bf16", seed=2),
    # head_dim 64, many blocks
    "g4_d64_many_blocks": W("g4_d64", 1, 8, 2, 64, 1024, 128, 128, 40, 1, "bf16", seed=8),
    # fp32 path, anchor shorter than the block
    "f32_gqa_d128": W("f32_gqa", 1, 4, 2, 128, 130, 64, 10, 3, 2, "f32", seed=7),
    "tiny_f32": syn.WORKLOADS["tiny_f32"],
}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")


def test_kv_write_rope_bit_exact():
    """K rows rotated at their cache row, in pieces; V copied; other rows untouched."""
    _need_gpu()
    for dtype, d in (("bf16", 128), ("bf16", 64), ("f32", 64)):
        w = W("rope_layout", 2, 6, 3, d, 150, 64, 64, 9, 0, dtype, seed=9)
        p = Pipeline(w, threads=1)
        rope = p.rope(sa.STAR_ROPE_ORIGINAL)
        p.write_context_rope(rope)
        sa.star_kv_write_rope(p.desc, p.k_cache, p.v_cache, w.ctx_len,
                              p.k_query[:, :4].contiguous(), p.v_query[:, :4].contiguous(), 4, rope)
        torch.cuda.synchronize()
        R = -(-(w.ctx_len + w.tail_cap) // 64) * 64
        raw = np.uint16 if dtype == "bf16" else np.uint32
        iv = torch.int16 if dtype == "bf16" else torch.int32
        kc = p.k_cache.view(iv).cpu().numpy().view(raw).reshape(w.batch, w.n_kv_heads, R, d)
        vc = p.v_cache.view(iv).cpu().numpy().view(raw).reshape(w.batch, w.n_kv_heads, R // 64, d, 64)
        k_in = np.concatenate([p.inputs["k_ctx"], p.inputs["k_tail"][:, :4]], axis=1)
        v_in = np.concatenate([p.inputs["v_ctx"], p.inputs["v_tail"][:, :4]], axis=1).view(raw)
        n = w.ctx_len + 4
        c, sn = p.rope_host
        kx = syn.to_f64(k_in, dtype)                               # [B, n, Hkv, d]
        cr, sr = c[:n][None, :, None, :], sn[:n][None, :, None, :]
        if dtype == "bf16":
            want = orc.rope_rotate_bf16(kx, cr, sr).astype(np.float32).view(np.uint32)
            want = (want >> 16).astype(np.uint16)
        else:
            want = orc.rope_rotate_f32(kx, cr, sr).view(np.uint32)
        nan = 0x7FC0 if dtype == "bf16" else np.float32(np.nan).view(np.uint32)
        for s in range(w.batch):
            for g in range(w.n_kv_heads):
                assert np.array_equal(kc[s, g, :n], want[s, :, g]), (dtype, d, s, g)
                vt = vc[s, g].transpose(0, 2, 1).reshape(R, d)
                assert np.array_equal(vt[:n], v_in[s, :, g]), (dtype, d, s, g)
                assert np.all(kc[s, g, n:] == nan) and np.all(vt[n:] == nan)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(CASES))
def test_phase1_rope_against_oracle(name, mode):
    _need_gpu()
    w = CASES[name]
    p = Pipeline(w, threads=4)
    rope = p.rope(MODES[mode])
    p.write_context_rope(rope)
    o = to_host_f64(p.phase1_rope(rope))
    x = {k: syn.to_f64(v, w.dtype) for k, v in p.inputs.items()}
    c, sn = (t.astype(np.float64) for t in p.rope_host)
    sc = orc.resolve_scale(w.head_dim, 0.0)
    ref = orc.phase1_rope(x["q_ctx"], x["k_ctx"], x["v_ctx"], w.block_len, w.anchor_len, sc, c, sn,
                          ORC_MODE[MODES[mode]])
    err = float(np.abs(o - ref).max())
    print(f"{name} {mode}: phase-1 rope max-abs error {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["gqa4_d128_ragged", "g1_unaligned_a_lt_b", "f32_gqa_d128"])
def test_phase1_rope_modes_and_identity_tables(name):
    """Block 0 has no anchor: both modes give the same bits there; with the
    anchor shorter than the block (or past block 1) the adjacent ids change
    the result; with identity tables (cos 1, sin 0) the rotary call gives
    plain phase 1 (bf16: the same bits in the original mode; in the adjacent
    mode the anchor's partial tile is summed earlier, so to the last bit;
    fp32: the same bits in both modes, since one kernel takes the same slices
    in the same order and the turned-back scores equal the plain ones)."""
    _need_gpu()
    w = CASES[name]
    p = Pipeline(w, threads=4)
    p.write_context()
    plain = p.phase1().clone()
    c = torch.ones(w.ctx_len + w.tail_cap, w.head_dim // 2, dtype=torch.float32, device="cuda")
    z = torch.zeros_like(c)
    iv = torch.int32 if w.dtype == "f32" else torch.int16
    for mname, mode in MODES.items():
        ident = sa.make_rope(c, z, mode)
        sa.star_kv_write_rope(p.desc, p.k_cache, p.v_cache, 0, p.dev["k_ctx"], p.dev["v_ctx"],
                              w.ctx_len, ident)
        got = p.phase1_rope(ident).clone()
        if w.dtype == "f32" or mname == "original":  # the same tiles in the same order
            assert torch.equal(got.view(iv), plain.view(iv))
        else:  # the anchor's partial tile comes before the block: another summation order
            err = float((got.float() - plain.float()).abs().max())
            assert err <= 2.0 ** -7 * float(plain.float().abs().max()) + 1e-6, err
    outs = {}
    for mname, mode in MODES.items():
        rope = p.rope(mode)
        p.write_context_rope(rope)
        outs[mname] = p.phase1_rope(rope).clone()
    torch.cuda.synchronize()
    b = w.block_len
    a, o = outs["original"], outs["adjacent"]
    assert torch.equal(a[:, :b].float(), o[:, :b].float())
    assert not torch.equal(a[:, b:].float(), o[:, b:].float())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", list(MODES))
def test_phase1_rope_full_size_32k_sampled(mode):
    """The 32K workload (8 blocks of 4096, anchor = block) at full size, both
    modes: sampled rows (block edges of the first, second, a middle and the
    last block, plus random rows) against the oracle."""
    _need_gpu()
    w = syn.workload("llama8b_32k")
    p = Pipeline(w, threads=16, fill_nan=False)
    rope = p.rope(MODES[mode])
    p.write_context_rope(rope)
    o = p.phase1_rope(rope)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = set()
    for i in sorted({0, 1, 2, w.n_blocks // 2, w.n_blocks - 1}):
        lo, hi = i * w.block_len, min((i + 1) * w.block_len, w.ctx_len)
        rows.update(r for r in (lo, lo + 1, lo + 63, lo + 64, (lo + hi) // 2, hi - 1) if lo <= r < hi)
    rows.update(int(x) for x in rng.integers(0, w.ctx_len, size=6))
    rows = sorted(rows)
    og = to_host_f64(o[0, rows])
    x = p.inputs
    c, sn = (t.astype(np.float64) for t in p.rope_host)
    sc = orc.resolve_scale(w.head_dim, 0.0)
    G = w.group
    qr = syn.to_f64(x["q_ctx"][0, rows], w.dtype)
    err = 0.0
    for g in range(w.n_kv_heads):
        K = syn.to_f64(x["k_ctx"][0, :, g], w.dtype)
        V = syn.to_f64(x["v_ctx"][0, :, g], w.dtype)
        ref = orc.phase1_rope_rows_one_head(qr[:, g * G:(g + 1) * G], K, V, rows, w.block_len,
                                            w.anchor_len, sc, c, sn, ORC_MODE[MODES[mode]])
        err = max(err, float(np.abs(og[:, g * G:(g + 1) * G] - ref).max()))
    print(f"32K rope {mode}: {len(rows)} rows, max-abs error {err:.3e}")
    assert err <= TOL["bf16"]
