"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` takes the oracle module and raises AssertionError when it
disagrees with a library routine, a closed form, brute force or an invariant
that the pages fix. The same functions run against the real oracle
(``test_oracle_pins.py``) and against copies with planted mistakes
(``test_oracle_mutations.py``), so each mistake must trip at least one pin.

Library routines used as independent references: torch's
``scaled_dot_product_attention`` (fp64, CPU, its own causal mask, default
scale and GQA head expansion) and ``torch.logsumexp``.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B, L, Hq, Hkv, d, scale_k=1.0):
    r = _rng(seed)
    q = r.standard_normal((B, L, Hq, d))
    k = r.standard_normal((B, L, Hkv, d)) * scale_k
    v = r.standard_normal((B, L, Hkv, d))
    return q, k, v


def _sdpa(q, k, v, causal=False, mask=None):
    """torch SDPA on token-major [B, T, H, d] float64 arrays (default scale)."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                       enable_gqa=(tq.shape[1] != tk.shape[1]))
    return o.numpy().transpose(0, 2, 1, 3)


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _scale(orc, d):
    return orc.resolve_scale(d, 0.0)


# ------------------------------------------------------------------ phase 1

def pin_phase1_one_block_is_causal_attention(orc):
    """With a single block, Star Attention phase 1 is full causal attention."""
    B, L, Hq, Hkv, d = 2, 13, 4, 2, 8
    q, k, v = _qkv(1, B, L, Hq, Hkv, d)
    for b in (13, 16, 64):
        o = orc.phase1(q, k, v, b, min(5, b), _scale(orc, d))
        _close(o, _sdpa(q, k, v, causal=True), what=f"one block b={b}")


def pin_phase1_block_is_causal_attention_over_anchor_concat(orc):
    """Block i >= 1 = causal attention over [anchor ; block i], block rows kept.

    The anchor (first a rows of the context) sits in front of the block and
    attention is causal over that concatenation.
    """
    B, L, Hq, Hkv, d = 1, 23, 4, 1, 8
    q, k, v = _qkv(2, B, L, Hq, Hkv, d)
    for b, a in ((6, 6), (6, 4), (5, 1), (8, 3)):
        o = orc.phase1(q, k, v, b, a, _scale(orc, d))
        for i in range(-(-L // b)):
            lo, hi = i * b, min((i + 1) * b, L)
            if i == 0:
                ref = _sdpa(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], causal=True)
            else:
                cat = lambda x: np.concatenate([x[:, :a], x[:, lo:hi]], axis=1)
                ref = _sdpa(cat(q), cat(k), cat(v), causal=True)[:, a:]
            _close(o[:, lo:hi], ref, what=f"block {i} (b={b}, a={a})")


def pin_phase1_second_block_is_exact_when_anchor_is_whole_block(orc):
    """With a = b the anchor is the whole first block, so block 1 is exact."""
    B, L, Hq, Hkv, d = 1, 20, 2, 2, 4
    q, k, v = _qkv(3, B, L, Hq, Hkv, d)
    b = 7
    o = orc.phase1(q, k, v, b, b, _scale(orc, d))
    full = _sdpa(q[:, :2 * b], k[:, :2 * b], v[:, :2 * b], causal=True)
    _close(o[:, :2 * b], full, what="blocks 0-1 with a=b")


def pin_phase1_uniform_scores_closed_form(orc):
    """K = 0 makes every visible key equally weighted: o(r) = mean of V over S1(r).

    |S1(r)| = a + (r - i*b + 1) for i >= 1 and r + 1 in block 0.
    """
    B, L, Hq, Hkv, d = 1, 17, 1, 1, 3
    r_ = _rng(4)
    q = r_.standard_normal((B, L, Hq, d))
    k = np.zeros((B, L, Hkv, d))
    v = r_.standard_normal((B, L, Hkv, d))
    b, a = 5, 3
    o = orc.phase1(q, k, v, b, a, 0.7)
    for r in range(L):
        i = r // b
        vis = (list(range(a)) if i else []) + list(range(i * b, r + 1))
        assert len(vis) == (a + r - i * b + 1 if i else r + 1)
        _close(o[0, r, 0], v[0, vis, 0].mean(axis=0), what=f"uniform row {r}")


def pin_phase1_blocks_are_independent(orc):
    """Changing a block other than 0 and i leaves block i's output bit-identical.

    Hosts do not communicate in phase 1 (paperhub.cn reply to dKGV point 1).
    """
    B, L, Hq, Hkv, d = 1, 24, 2, 1, 4
    q, k, v = _qkv(5, B, L, Hq, Hkv, d)
    b, a = 6, 6
    o = orc.phase1(q, k, v, b, a, _scale(orc, d))
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:, 12:18] += 3.0
    v2[:, 12:18] -= 1.5
    q2[:, 12:18] *= -1.0
    o2 = orc.phase1(q2, k2, v2, b, a, _scale(orc, d))
    for lo, hi in ((0, 6), (6, 12), (18, 24)):
        assert np.array_equal(o[:, lo:hi], o2[:, lo:hi]), f"block [{lo},{hi}) changed"
    assert not np.array_equal(o[:, 12:18], o2[:, 12:18])


def pin_phase1_row_agrees_with_brute_force(orc):
    """phase1 and phase1_row against pure-Python loops (math.fsum)."""
    B, L, Hq, Hkv, d = 1, 10, 4, 2, 4
    q, k, v = _qkv(6, B, L, Hq, Hkv, d)
    b, a = 4, 3
    sc = _scale(orc, d)
    bf = np.array(orc.brute_force_phase1(q.tolist(), k.tolist(), v.tolist(), b, a, sc))
    _close(orc.phase1(q, k, v, b, a, sc), bf, what="phase1 vs brute force")
    for r in range(L):
        for h in range(Hq):
            _close(orc.phase1_row(q, k, v, 0, r, h, b, a, sc), bf[0, r, h],
                   what=f"phase1_row r={r} h={h}")


def pin_brute_force_is_sdpa(orc):
    """The brute force itself reproduces SDPA on one block (so it is no echo)."""
    B, L, Hq, Hkv, d = 1, 6, 2, 1, 3
    q, k, v = _qkv(7, B, L, Hq, Hkv, d)
    bf = np.array(orc.brute_force_phase1(q.tolist(), k.tolist(), v.tolist(), 6, 6,
                                         1.0 / math.sqrt(d)))
    _close(bf, _sdpa(q, k, v, causal=True), what="brute force vs SDPA")


# ------------------------------------------------------------------ phase 2

def _tail_case(seed, B=2, L=18, T=5, Hq=4, Hkv=2, d=8, scale_k=1.0):
    q, k, v = _qkv(seed, B, L + T, Hq, Hkv, d, scale_k)
    return q[:, L:], k, v, L, T


def _causal_tail_mask(L, T):
    m = np.zeros((T, L + T), dtype=bool)
    for j in range(T):
        m[j, :L + j + 1] = True
    return m


def pin_phase2_dense_is_masked_sdpa(orc):
    """Dense phase 2 = SDPA with the tail's causal mask; lse = torch.logsumexp."""
    qt, k, v, L, T = _tail_case(8)
    pos = [L + j for j in range(T)]
    d = k.shape[-1]
    o, lse = orc.phase2_dense(qt, k, v, pos, _scale(orc, d))
    mask = _causal_tail_mask(L, T)
    _close(o, _sdpa(qt, k, v, mask=mask), what="phase2 vs SDPA")
    tq = torch.from_numpy(qt.transpose(0, 2, 1, 3).copy())
    tk = torch.from_numpy(k.transpose(0, 2, 1, 3).copy()).repeat_interleave(2, dim=1)
    s = torch.matmul(tq, tk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(~torch.from_numpy(mask), -math.inf)
    ref = torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1)
    _close(lse, ref, what="lse vs torch.logsumexp")


def pin_phase2_partials_merge_to_dense(orc):
    """Per-host partials + exact merge = dense attention, for any block size."""
    qt, k, v, L, T = _tail_case(9, scale_k=3.0)
    pos = [L + j for j in range(T)]
    sc = _scale(orc, k.shape[-1])
    o, lse = orc.phase2_dense(qt, k, v, pos, sc)
    for b in (1, 4, 5, 18, 40):
        o2, lse2 = orc.phase2_via_partials(qt, k, v, pos, L, b, L + T, sc)
        _close(o2, o, what=f"partials b={b}")
        _close(lse2, lse, what=f"partial lse b={b}")


def pin_phase2_pieces_cover_cache_once(orc):
    """The hosts' shares tile [0, kv_len) exactly once, blocks then the tail."""
    for L, b, kv in ((18, 4, 23), (16, 4, 16), (7, 7, 9), (10, 3, 11)):
        pcs = orc.phase2_pieces(L, b, kv)
        cover = np.zeros(kv, dtype=int)
        for lo, hi in pcs:
            assert lo < hi
            cover[lo:hi] += 1
        assert (cover == 1).all(), (L, b, kv, pcs)
        assert all(hi <= L or lo >= L for lo, hi in pcs), "a piece straddles the tail"
        assert sum(1 for lo, hi in pcs if hi <= L) == -(-L // b)


def pin_merge_identities(orc):
    """One piece: identity. Permuting pieces: invariant. -inf piece: weight 0."""
    r = _rng(10)
    o1 = r.standard_normal(6)
    o, l = orc.lse_merge(o1[None], np.array([1.25]))
    _close(o, o1, what="single piece o")
    _close(l, 1.25, what="single piece lse")
    op = r.standard_normal((5, 6))
    lp = r.standard_normal(5) * 4
    o, l = orc.lse_merge(op, lp)
    perm = r.permutation(5)
    o2, l2 = orc.lse_merge(op[perm], lp[perm])
    _close(o2, o, what="permuted o")
    _close(l2, l, what="permuted lse")
    o3, l3 = orc.lse_merge(np.vstack([op, r.standard_normal((1, 6))]),
                           np.concatenate([lp, [-math.inf]]))
    _close(o3, o, what="-inf piece o")
    _close(l3, l, what="-inf piece lse")
    # closed form: two pieces with lse ln1 and ln3 -> weights 1/4, 3/4
    o4, l4 = orc.lse_merge(np.array([[4.0, 0.0], [0.0, 4.0]]), np.array([0.0, math.log(3.0)]))
    _close(o4, [1.0, 3.0], what="closed-form merge")
    _close(l4, math.log(4.0), what="closed-form merge lse")


def pin_attend_closed_form(orc):
    """Two keys with scaled scores 0 and ln 3: weights 1/4 and 3/4, lse = ln 4."""
    sc = 0.5
    q = np.array([1.0, 0.0])
    K = np.array([[0.0, 5.0], [math.log(3.0) / sc, -2.0]])
    V = np.array([[8.0, -4.0], [0.0, 4.0]])
    o, l = orc.attend(q, K, V, sc)
    _close(o, [2.0, 2.0], what="closed-form attend")
    _close(l, math.log(4.0), what="closed-form lse")
    # equal scores: lse = s + ln n, o = mean
    K = np.tile(np.array([[0.3, 0.1]]), (7, 1))
    V = _rng(11).standard_normal((7, 2))
    o, l = orc.attend(q, K, V, sc)
    _close(o, V.mean(axis=0), what="uniform attend")
    _close(l, sc * 0.3 + math.log(7.0), what="uniform lse")


def pin_constant_values_pass_through(orc):
    """V == c makes every output c, in both phases (weights sum to one)."""
    B, L, Hq, Hkv, d = 1, 15, 2, 1, 3
    q, k, _ = _qkv(12, B, L, Hq, Hkv, d, scale_k=5.0)
    v = np.full((B, L, Hkv, d), -2.5)
    _close(orc.phase1(q, k, v, 4, 2, 0.9), np.full((B, L, Hq, d), -2.5), what="phase1 const")
    o, _ = orc.phase2_via_partials(q[:, 10:], k, v, list(range(10, 15)), 10, 3, 15, 0.9)
    _close(o, np.full((B, 5, Hq, d), -2.5), what="phase2 const")


def pin_phase2_brute_force(orc):
    """Dense phase 2 and its partials against scalar loops."""
    qt, k, v, L, T = _tail_case(13, B=1, L=7, T=3, Hq=2, Hkv=1, d=3)
    pos = [L + j for j in range(T)]
    sc = 0.8
    bo, bl = orc.brute_force_phase2(qt.tolist(), k.tolist(), v.tolist(), pos, sc)
    o, l = orc.phase2_dense(qt, k, v, pos, sc)
    _close(o, np.array(bo), what="phase2 brute o")
    _close(l, np.array(bl), what="phase2 brute lse")
    o2, l2 = orc.phase2_via_partials(qt, k, v, pos, L, 3, L + T, sc)
    _close(o2, np.array(bo), what="phase2 partial brute o")
    _close(l2, np.array(bl), what="phase2 partial brute lse")


def pin_decode_equals_one_causal_call(orc):
    """Token-by-token decode == one phase-2 call over all tail rows (causal tail)."""
    B, L, T, Hq, Hkv, d = 1, 12, 6, 4, 2, 4
    q, k, v = _qkv(14, B, L + T, Hq, Hkv, d)
    sc = _scale(orc, d)
    O, LSE = orc.decode_loop(q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:], 2, sc)
    o, l = orc.phase2_dense(q[:, L:], k, v, [L + j for j in range(T)], sc)
    _close(O, o, what="decode o")
    _close(LSE, l, what="decode lse")
    _close(O, _sdpa(q[:, L:], k, v, mask=_causal_tail_mask(L, T)), what="decode vs SDPA")


def pin_empty_host_reply(orc):
    """A host whose rows all lie after the query returns (0, -inf)."""
    K = _rng(15).standard_normal((10, 3))
    o, l = orc.phase2_partial(np.ones(3), K, K, 4, 6, 10, 1.0)
    assert l == -math.inf and np.all(o == 0.0)


def pin_scale_default(orc):
    """softmax_scale 0 means 1/sqrt(head_dim); a non-zero value is used as is."""
    assert abs(orc.resolve_scale(64, 0.0) - 0.125) < 1e-15
    assert abs(orc.resolve_scale(128, 0.0) - 1 / math.sqrt(128)) < 1e-15
    assert orc.resolve_scale(128, 0.3) == 0.3


def pin_sampled_row_forms_match_sdpa(orc):
    """The per-kv-head sampled-row forms against SDPA (GQA) on every row."""
    B, L, Hq, Hkv, d = 1, 26, 6, 2, 8
    q, k, v = _qkv(16, B, L, Hq, Hkv, d)
    G = Hq // Hkv
    sc = _scale(orc, d)
    b, a = 8, 5
    rows = list(range(L))
    for g in range(Hkv):
        o = orc.phase1_rows_one_head(q[0, rows, g * G:(g + 1) * G], k[0, :, g], v[0, :, g],
                                     rows, b, a, sc)
        for i in range(-(-L // b)):
            lo, hi = i * b, min((i + 1) * b, L)
            if i == 0:
                ref = _sdpa(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], causal=True)
            else:
                cat = lambda x: np.concatenate([x[:, :a], x[:, lo:hi]], axis=1)
                ref = _sdpa(cat(q), cat(k), cat(v), causal=True)[:, a:]
            _close(o[lo:hi], ref[0, :, g * G:(g + 1) * G], what=f"sampled phase1 g={g} block {i}")
    qt, k2, v2, L2, T = _tail_case(17, B=1, Hq=6, Hkv=2)
    pos = [L2 + j for j in range(T)]
    ref = _sdpa(qt, k2, v2, mask=_causal_tail_mask(L2, T))
    tq = torch.from_numpy(qt.transpose(0, 2, 1, 3).copy())
    tk = torch.from_numpy(k2.transpose(0, 2, 1, 3).copy()).repeat_interleave(3, dim=1)
    s = torch.matmul(tq, tk.transpose(-1, -2)) * sc
    s = s.masked_fill(~torch.from_numpy(_causal_tail_mask(L2, T)), -math.inf)
    lref = torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1)
    for g in range(2):
        o, l = orc.phase2_rows_one_head(qt[0, :, g * 3:(g + 1) * 3], k2[0, :, g], v2[0, :, g],
                                        pos, sc)
        _close(o, ref[0, :, g * 3:(g + 1) * 3], what=f"sampled phase2 g={g}")
        _close(l, lref[0, :, g * 3:(g + 1) * 3], what=f"sampled phase2 lse g={g}")


def pin_block_rows_form_matches_sdpa(orc):
    """The block-batched sampled-row form against SDPA over [anchor ; block]
    (block 0: plain causal attention), on every block, with a ragged last
    block, a < b, GQA 3:1, rows in any order and repeated."""
    B, L, Hq, Hkv, d = 1, 29, 6, 2, 8
    q, k, v = _qkv(18, B, L, Hq, Hkv, d)
    G = Hq // Hkv
    sc = _scale(orc, d)
    b, a = 8, 5
    rng = np.random.default_rng(3)
    for i in range(-(-L // b)):
        lo, hi = i * b, min((i + 1) * b, L)
        rows = list(rng.permutation(np.arange(lo, hi))) + [lo]
        if i == 0:
            ref = _sdpa(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], causal=True)
        else:
            cat = lambda x: np.concatenate([x[:, :a], x[:, lo:hi]], axis=1)
            ref = _sdpa(cat(q), cat(k), cat(v), causal=True)[:, a:]
        for g in range(Hkv):
            o = orc.phase1_block_rows_one_head(q[0, rows, g * G:(g + 1) * G], k[0, :, g],
                                               v[0, :, g], rows, b, a, sc)
            _close(o, ref[0, [r - lo for r in rows], g * G:(g + 1) * G],
                   what=f"block rows g={g} block {i}")


# ------------------------------------------------------------------ rotary embedding

def _angles(n_pos, d, theta=10000.0, offset=0):
    """Angle table ``[n_pos, d/2]``: (offset + pos) * theta^(-2i/d)."""
    i = np.arange(d // 2, dtype=np.float64)
    return (offset + np.arange(n_pos, dtype=np.float64))[:, None] * theta ** (-2.0 * i / d)


def _rot_complex(x, ang):
    """Half-split rotation written as complex multiplication: element i and
    element i + d/2 are the real and imaginary parts of one number, turned by
    the angle."""
    h = x.shape[-1] // 2
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def pin_rope_is_complex_multiplication(orc):
    x = _rng(40).standard_normal((7, 16))
    ang = _angles(7, 16) * 3.1
    _close(orc.rope_rotate(x, np.cos(ang), np.sin(ang)), _rot_complex(x, ang), 1e-12, "rope")


def pin_rope_scores_depend_on_relative_position(orc):
    """<R(p) q, R(p') k> depends only on p - p' (tables from true angles)."""
    r = _rng(41)
    q, k = r.standard_normal(16), r.standard_normal(16)
    a0, a1 = _angles(64, 16), _angles(64, 16, offset=1000)
    for p, pk in ((9, 2), (40, 40), (3, 50)):
        s0 = orc.rope_rotate(q, np.cos(a0[p]), np.sin(a0[p])) @ \
            orc.rope_rotate(k, np.cos(a0[pk]), np.sin(a0[pk]))
        s1 = orc.rope_rotate(q, np.cos(a1[p]), np.sin(a1[p])) @ \
            orc.rope_rotate(k, np.cos(a1[pk]), np.sin(a1[pk]))
        _close(s0, s1, 1e-9, "relative position")


def pin_rope_bf16_is_torch_fp32_then_bf16(orc):
    """The bf16 form equals torch's float32 arithmetic (separate multiply and
    add on the CPU) followed by torch's bfloat16 conversion (nearest, ties to
    even), on bf16 inputs, including values on rounding ties."""
    r = _rng(42)
    x = torch.from_numpy(r.standard_normal((33, 32)).astype(np.float32)).to(torch.bfloat16).float()
    ang = _angles(33, 32, theta=500000.0) * 1.7
    c = torch.from_numpy(np.cos(ang).astype(np.float32))
    sn = torch.from_numpy(np.sin(ang).astype(np.float32))
    lo, hi = x[:, :16], x[:, 16:]
    y32 = torch.cat([lo * c - hi * sn, hi * c + lo * sn], dim=1)
    _close(orc.rope_rotate_f32(x.numpy(), c.numpy(), sn.numpy()), y32.double().numpy(), 0.0,
           "rope f32")
    y = y32.to(torch.bfloat16).double()
    _close(orc.rope_rotate_bf16(x.numpy(), c.numpy(), sn.numpy()), y.numpy(), 0.0, "rope bf16")
    # cancellation: rounding each product to float32 gives 2^-23, the exact
    # difference 2^-23 (1 + 2^-7); both are bf16 values
    xc = torch.tensor([[1.0078125, 1.0078125]], dtype=torch.float32)
    cc = torch.tensor([[1.0 + 3 * 2.0 ** -23]], dtype=torch.float32)
    sc_ = torch.tensor([[1.0 + 2.0 ** -22]], dtype=torch.float32)
    yc = (xc[:, :1] * cc - xc[:, 1:] * sc_).to(torch.bfloat16).double()
    assert float(yc) == 2.0 ** -23
    _close(orc.rope_rotate_bf16(xc.numpy(), cc.numpy(), sc_.numpy())[:, :1], yc.numpy(), 0.0,
           "cancellation")
    # exact ties: 1 + 2^-8 (tie, even below) and 1 + 3 * 2^-8 (tie, even above)
    t = np.array([[1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 0.0, 0.0]], dtype=np.float32)
    one, zero = np.ones((1, 2), np.float32), np.zeros((1, 2), np.float32)
    _close(orc.rope_rotate_bf16(t, one, zero)[0, :2], [1.0, 1.0 + 2.0 ** -6], 0.0, "ties")


def _rope_case(seed, L=21, b=8, a=5, Hq=4, Hkv=2, d=8):
    q, k, v = _qkv(seed, 2, L, Hq, Hkv, d)
    ang = _angles(L, d) * 0.9
    return q, k, v, b, a, ang


def pin_phase1_rope_identity_table_is_phase1(orc):
    q, k, v, b, a, ang = _rope_case(43)
    L, h = q.shape[1], q.shape[3] // 2
    one, zero = np.ones((L, h)), np.zeros((L, h))
    sc = _scale(orc, q.shape[3])
    for mode in (orc.ROPE_ORIGINAL, orc.ROPE_ADJACENT):
        _close(orc.phase1_rope(q, k, v, b, a, sc, one, zero, mode),
               orc.phase1(q, k, v, b, a, sc), 1e-12, f"identity table, mode {mode}")


def pin_phase1_rope_original_is_phase1_of_rotated_inputs(orc):
    """ORIGINAL: every row keeps its context position, so the result is plain
    phase 1 on inputs rotated beforehand (by the complex form)."""
    q, k, v, b, a, ang = _rope_case(44)
    sc = _scale(orc, q.shape[3])
    qr = _rot_complex(q, ang[None, :, None, :])
    kr = _rot_complex(k, ang[None, :, None, :])
    _close(orc.phase1_rope(q, k, v, b, a, sc, np.cos(ang), np.sin(ang), orc.ROPE_ORIGINAL),
           orc.phase1(qr, kr, v, b, a, sc), 1e-12, "original")


def pin_phase1_rope_adjacent_brute_force(orc):
    """ADJACENT, row by row from the stated position ids: anchor row j of
    block i >= 1 at position i*b - a + j, every other row at its own, each
    query attending to the anchor then causally to its block."""
    q, k, v, b, a, ang = _rope_case(45)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    sc = _scale(orc, d)
    ext = _angles(2 * L, d) * 0.9  # the same schedule, positions up to 2L
    got = orc.phase1_rope(q, k, v, b, a, sc, np.cos(ext), np.sin(ext), orc.ROPE_ADJACENT)
    for s in range(B):
        for r in range(L):
            i = r // b
            keys = list(range(i * b, r + 1))
            pos = list(keys)
            if i > 0:
                keys = list(range(a)) + keys
                pos = [i * b - a + j for j in range(a)] + pos
            for h in range(Hq):
                g = h // (Hq // Hkv)
                qq = _rot_complex(q[s, r, h], ext[r])
                kk = np.stack([_rot_complex(k[s, kr, g], ext[p]) for kr, p in zip(keys, pos)])
                w = np.exp(sc * (kk @ qq) - np.max(sc * (kk @ qq)))
                _close(got[s, r, h], (w @ v[s, keys, g]) / w.sum(), 1e-12, f"row {r}")


def pin_phase1_rope_adjacent_is_query_shift(orc):
    """Rotations compose, so ADJACENT scores for block i equal those of keys
    kept at their own positions with the query turned back by i*b - a for the
    anchor part: the identity the kernel relies on, checked here on the
    oracle against a run that applies it explicitly."""
    q, k, v, b, a, ang = _rope_case(46, L=24, b=8, a=8)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    sc = _scale(orc, d)
    ext = _angles(2 * L, d) * 0.7
    got = orc.phase1_rope(q, k, v, b, a, sc, np.cos(ext), np.sin(ext), orc.ROPE_ADJACENT)
    for s in range(B):
        for r in range(b, L):
            i, delta = r // b, (r // b) * b - a
            for h in range(Hq):
                g = h // (Hq // Hkv)
                qa = _rot_complex(q[s, r, h], ext[r - delta])
                ql = _rot_complex(q[s, r, h], ext[r])
                ka = np.stack([_rot_complex(k[s, j, g], ext[j]) for j in range(a)])
                kl = np.stack([_rot_complex(k[s, j, g], ext[j]) for j in range(i * b, r + 1)])
                sco = sc * np.concatenate([ka @ qa, kl @ ql])
                w = np.exp(sco - sco.max())
                vv = np.concatenate([v[s, :a, g], v[s, i * b:r + 1, g]])
                _close(got[s, r, h], (w @ vv) / w.sum(), 1e-12, f"shift row {r}")


def pin_phase1_rope_sampled_rows_match_full(orc):
    """The sampled-row form equals the full one (itself pinned above) on every
    row, both modes."""
    q, k, v, b, a, ang = _rope_case(47, L=21, b=8, a=5, Hq=4, Hkv=2)
    L = q.shape[1]
    sc = _scale(orc, q.shape[3])
    ext = _angles(2 * L, q.shape[3]) * 1.3
    rows = list(range(L))
    for mode in (orc.ROPE_ORIGINAL, orc.ROPE_ADJACENT):
        full = orc.phase1_rope(q, k, v, b, a, sc, np.cos(ext), np.sin(ext), mode)
        for s in range(q.shape[0]):
            for g in range(k.shape[2]):
                hs = slice(2 * g, 2 * g + 2)
                got = orc.phase1_rope_rows_one_head(q[s, :, hs], k[s, :, g], v[s, :, g], rows, b,
                                                    a, sc, np.cos(ext), np.sin(ext), mode)
                _close(got, full[s, :, hs], 1e-12, f"sampled rope rows, mode {mode}")


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
