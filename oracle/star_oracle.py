"""Plain fp64 CPU oracle for the Star Attention two-phase attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` use it. It shares no code, header,
table or helper with the HIP library; it receives the same generator output
(bf16 bit patterns widened exactly, or fp32 values) and computes in float64.

Sources (all pages carry the title "Star Attention: Efficient LLM Inference
over Long Sequences"):

* hotaipapers.com summary page, Abstract, and podcast transcript: the Phase 1
  description (context cut into blocks, one per host; every block after the
  first is prefixed with an anchor block that copies the first block; blocks
  run in parallel with local attention only) and the Phase 2 description
  (the query goes to every host; each host attends over its own cached KV and
  sends back one vector and one scalar; the query host aggregates them into
  global attention, appends to its KV cache and repeats token by token).
* proceedings.mlr.press (PMLR 267) page, Abstract: phase 2 query and response
  tokens attend to all earlier cached tokens.
* paperhub.cn rebuttal page: reply to reviewer EMsM, point 5, and reply to
  x5MA, point 1 (phase 1 attention is causal; the anchor is the first context
  block and is at most one block long); reply to dnhh, point 2 (phase 2 is
  dense over the full KV cache built in phase 1); replies to dnhh, points 1
  and 3, and to dKGV, point 1 (no communication between hosts in phase 1).

Readings where the pages are silent are listed with each function; the
same list is kept with the project's design notes.

Every function here has at least one pin in ``tests/test_oracle_pins.py``
that does not reuse this code (library routines, closed forms, brute force,
invariants); ``tests/test_oracle_mutations.py`` plants plausible mistakes in a
copy of this file and checks that the pins catch each one.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Shared definitions
# --------------------------------------------------------------------------

def resolve_scale(head_dim: int, softmax_scale: float) -> float:
    """Softmax temperature applied to q.k.

    The pages never print the scale (reading: the usual 1/sqrt(head_dim) of
    the dot-product attention the models were trained with; a non-zero value
    overrides it).
    """
    return 1.0 / math.sqrt(head_dim) if softmax_scale == 0.0 else float(softmax_scale)


def kv_head(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head serving query head ``h`` under grouped-query attention.

    The pages do not discuss GQA (reading: consecutive query heads share a KV
    head, as in the Llama models the pages evaluate).
    """
    return h // (n_q_heads // n_kv_heads)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray,
           scale: float) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query over a set of key rows.

    Returns the normalised output ``sum_r w_r V[r]`` with
    ``w_r = exp(scale q.K[r]) / sum_r' exp(scale q.K[r'])`` and the natural-log
    log-sum-exp of the scaled scores. An empty key set gives ``(0, -inf)``.
    """
    d = V.shape[-1] if V.ndim == 2 else q.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(d, dtype=np.float64), -math.inf
    s = scale * (K @ q)
    m = float(s.max())
    e = np.exp(s - m)
    z = float(e.sum())
    return (e @ V) / z, m + math.log(z)


# --------------------------------------------------------------------------
# Phase 1: blockwise-local causal attention with the anchor block
# --------------------------------------------------------------------------

def phase1_key_rows(r: int, block_len: int, anchor_len: int) -> np.ndarray:
    """Context rows that context row ``r`` attends to in phase 1.

    Block ``i = r // block_len`` holds rows ``[i*b, (i+1)*b)``. Every block
    after the first sees the anchor (rows ``[0, a)`` of the first block)
    in front of itself, and causal attention inside the block, including
    the row itself (hotaipapers.com podcast, Phase 1; paperhub.cn reply to
    EMsM point 5: causal, anchor before the block). Block 0 has no anchor.
    """
    i = r // block_len
    local = np.arange(i * block_len, r + 1, dtype=np.int64)
    if i == 0:
        return local
    return np.concatenate([np.arange(anchor_len, dtype=np.int64), local])


def phase1_row(q_ctx: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
               seq: int, r: int, h: int, block_len: int, anchor_len: int,
               scale: float) -> np.ndarray:
    """Phase-1 output of one (sequence, context row, query head).

    Inputs are token-major float64 arrays ``[B, L, H, d]``.
    """
    Hq, Hkv = q_ctx.shape[2], k_ctx.shape[2]
    g = kv_head(h, Hq, Hkv)
    rows = phase1_key_rows(r, block_len, anchor_len)
    o, _ = attend(q_ctx[seq, r, h], k_ctx[seq, rows, g], v_ctx[seq, rows, g], scale)
    return o


def phase1(q_ctx: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
           block_len: int, anchor_len: int, scale: float) -> np.ndarray:
    """Phase-1 output for every context row: ``[B, L, Hq, d]`` float64.

    Block by block: the keys are the anchor rows followed by the block rows
    (block 0: only its own rows); a block row sees every anchor row and the
    block rows up to itself. One output per context token; the anchor's own
    rows are not recomputed for later blocks (reading: they would equal
    block 0's outputs, and the cache keeps each token once).
    """
    B, L, Hq, d = q_ctx.shape
    Hkv = k_ctx.shape[2]
    out = np.zeros((B, L, Hq, d), dtype=np.float64)
    n_blocks = -(-L // block_len)
    for s in range(B):
        for i in range(n_blocks):
            lo, hi = i * block_len, min((i + 1) * block_len, L)
            n_loc = hi - lo
            anc = np.arange(anchor_len) if i > 0 else np.arange(0)
            keys = np.concatenate([anc, np.arange(lo, hi)])
            # visible[r, j]: block row r sees key j
            visible = np.zeros((n_loc, keys.size), dtype=bool)
            visible[:, :anc.size] = True
            visible[:, anc.size:] = np.tril(np.ones((n_loc, n_loc), dtype=bool))
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                Q = q_ctx[s, lo:hi, h]
                K = k_ctx[s, keys, g]
                V = v_ctx[s, keys, g]
                S = scale * (Q @ K.T)
                S = np.where(visible, S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                out[s, lo:hi, h] = (E @ V) / E.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# Phase 2: sequence-global attention from per-host partials
# --------------------------------------------------------------------------

def phase2_pieces(ctx_len: int, block_len: int, kv_len: int) -> List[Tuple[int, int]]:
    """The hosts' shares of the phase-2 KV cache, as row ranges.

    One piece per context block (each context token cached once; the anchor
    copies are not part of the cache), then the query host's tail of query
    and generated tokens ``[ctx_len, kv_len)`` (hotaipapers.com podcast,
    Phase 2; paperhub.cn reply to dnhh point 2: the full KV state of
    phase 1). Empty tail is omitted.
    """
    pieces = [(lo, min(lo + block_len, ctx_len)) for lo in range(0, ctx_len, block_len)]
    if kv_len > ctx_len:
        pieces.append((ctx_len, kv_len))
    return pieces


def phase2_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: int,
                   lo: int, hi: int, scale: float) -> Tuple[np.ndarray, float]:
    """One host's reply for a query at absolute position ``pos``.

    The host holds cache rows ``[lo, hi)``; the query sees rows ``<= pos``
    (causal inside the tail: reading, since query and generated tokens are
    appended in order). The reply is the host-local normalised output (the
    vector) and its natural-log log-sum-exp (the scalar); hotaipapers.com
    podcast, Phase 2: one vector and one scalar per host.
    """
    top = min(hi, pos + 1)
    if top <= lo:
        return np.zeros(V.shape[-1], dtype=np.float64), -math.inf
    return attend(q, K[lo:top], V[lo:top], scale)


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, float]:
    """Query-host aggregation of per-host (vector, scalar) replies.

    Exact softmax renormalisation (the pages name the aggregation without a
    formula; reading: each partial's weight is exp(lse_h - lse) with
    ``lse = log sum_h exp(lse_h)``). Hosts with ``lse = -inf`` (no visible
    key) get weight zero. ``o_parts``: ``[S, d]``, ``lse_parts``: ``[S]``.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    if not finite.any():
        return np.zeros(o_parts.shape[-1], dtype=np.float64), -math.inf
    m = float(lse_parts[finite].max())
    w = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m), 0.0)
    z = float(w.sum())
    o = (w @ o_parts) / z
    return o, m + math.log(z)


def phase2_dense(q_rows: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                 positions: Sequence[int], scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dense global attention of query rows over the whole cache.

    ``q_rows``: ``[B, n, Hq, d]``; ``k_all``/``v_all``: ``[B, N, Hkv, d]`` with
    the context rows followed by the tail rows; query ``j`` sits at absolute
    position ``positions[j]`` and sees rows ``[0, positions[j]]`` (PMLR page,
    Abstract: attention over all earlier cached tokens). Returns
    ``(O [B, n, Hq, d], lse [B, n, Hq])``.
    """
    B, n, Hq, d = q_rows.shape
    Hkv = k_all.shape[2]
    O = np.zeros((B, n, Hq, d), dtype=np.float64)
    LSE = np.zeros((B, n, Hq), dtype=np.float64)
    for s in range(B):
        for j, p in enumerate(positions):
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                o, l = attend(q_rows[s, j, h], k_all[s, :p + 1, g], v_all[s, :p + 1, g], scale)
                O[s, j, h], LSE[s, j, h] = o, l
    return O, LSE


def phase2_via_partials(q_rows: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                        positions: Sequence[int], ctx_len: int, block_len: int,
                        kv_len: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Phase 2 as the pages run it: per-host partials, then the merge."""
    B, n, Hq, d = q_rows.shape
    Hkv = k_all.shape[2]
    pieces = phase2_pieces(ctx_len, block_len, kv_len)
    O = np.zeros((B, n, Hq, d), dtype=np.float64)
    LSE = np.zeros((B, n, Hq), dtype=np.float64)
    for s in range(B):
        for j, p in enumerate(positions):
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                parts = [phase2_partial(q_rows[s, j, h], k_all[s, :, g], v_all[s, :, g],
                                        p, lo, hi, scale) for lo, hi in pieces]
                o_p = np.stack([x[0] for x in parts])
                l_p = np.array([x[1] for x in parts])
                O[s, j, h], LSE[s, j, h] = lse_merge(o_p, l_p)
    return O, LSE


def decode_loop(q_tail: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
                k_tail: np.ndarray, v_tail: np.ndarray, n_query: int,
                scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Query step then token-by-token decode, as the query host runs it.

    The ``n_query`` query rows are appended to the cache and attend to it;
    then each pre-drawn decode row (there is no model, so the next token's
    q/k/v are inputs) is appended and attends to everything before it and
    itself (hotaipapers.com podcast, Phase 2: update the cache, repeat
    autoregressively). Returns outputs and lse for all tail rows, in order.
    """
    B, L, Hkv, d = k_ctx.shape
    T = q_tail.shape[1]
    k_all = np.concatenate([k_ctx, k_tail], axis=1)
    v_all = np.concatenate([v_ctx, v_tail], axis=1)
    O = np.zeros((B, T, q_tail.shape[2], d), dtype=np.float64)
    LSE = np.zeros((B, T, q_tail.shape[2]), dtype=np.float64)
    # query step: one call over the n_query rows
    o, l = phase2_dense(q_tail[:, :n_query], k_all[:, :L + n_query], v_all[:, :L + n_query],
                        [L + j for j in range(n_query)], scale)
    O[:, :n_query], LSE[:, :n_query] = o, l
    # decode: one row per step, cache grows by one
    for t in range(n_query, T):
        kv_len = L + t + 1
        o, l = phase2_dense(q_tail[:, t:t + 1], k_all[:, :kv_len], v_all[:, :kv_len],
                            [L + t], scale)
        O[:, t], LSE[:, t] = o[:, 0], l[:, 0]
    return O, LSE


# --------------------------------------------------------------------------
# Sampled rows of one kv head (for full-size checks): the same definitions,
# evaluated for a few rows with one matmul over the query heads sharing K/V.
# --------------------------------------------------------------------------

def _softmax_rows(S: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of scores S [h, n] (already scaled, -inf = masked) times V [n, d]."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    z = E.sum(axis=1, keepdims=True)
    return (E @ V) / z, (m + np.log(z))[:, 0]


def phase1_rows_one_head(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                         rows: Sequence[int], block_len: int, anchor_len: int,
                         scale: float) -> np.ndarray:
    """Phase-1 outputs of sampled context rows for the query heads of one kv head.

    ``q_rows``: ``[n, h, d]`` queries of rows ``rows[k]`` (h heads sharing this
    kv head); ``K``, ``V``: ``[L', d]`` context rows of the kv head (at least
    up to the largest sampled row). Key set as in ``phase1_key_rows``.
    Returns ``[n, h, d]``.
    """
    out = np.zeros(q_rows.shape, dtype=np.float64)
    for k, r in enumerate(rows):
        keys = phase1_key_rows(int(r), block_len, anchor_len)
        Kk = np.asarray(K[keys], dtype=np.float64)
        Vk = np.asarray(V[keys], dtype=np.float64)
        S = scale * (np.asarray(q_rows[k], dtype=np.float64) @ Kk.T)
        out[k], _ = _softmax_rows(S, Vk)
    return out


def phase1_block_rows_one_head(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                               rows: Sequence[int], block_len: int, anchor_len: int,
                               scale: float) -> np.ndarray:
    """Phase-1 outputs of sampled rows that all lie in one context block, for
    the query heads of one kv head, with one product over the block's key set.

    Same definition as ``phase1_rows_one_head`` (key set of
    ``phase1_key_rows``): the rows of block ``i`` share the anchor ``[0, a)``
    (for ``i >= 1``) and the block's rows up to the last sampled row; each
    row masks the block keys after itself. ``q_rows``: ``[n, h, d]``;
    ``K``, ``V``: ``[L', d]``. Returns ``[n, h, d]``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    i = int(rows[0]) // block_len
    assert (rows // block_len == i).all(), "rows of one block"
    lo, hi = i * block_len, int(rows.max()) + 1
    anc = np.arange(anchor_len if i > 0 else 0, dtype=np.int64)
    blk = np.arange(lo, hi, dtype=np.int64)
    keys = np.concatenate([anc, blk])
    Kk = np.asarray(K[keys], dtype=np.float64)
    Vk = np.asarray(V[keys], dtype=np.float64)
    q = np.asarray(q_rows, dtype=np.float64)
    n, h, d = q.shape
    S = scale * (q.reshape(n * h, d) @ Kk.T)                 # [n*h, |keys|]
    # block key j (row lo + j) is visible to row r when lo + j <= r
    visible = np.ones((n, len(keys)), dtype=bool)
    visible[:, len(anc):] = blk[None, :] <= rows[:, None]
    S = np.where(np.repeat(visible, h, axis=0), S, -np.inf)
    out, _ = _softmax_rows(S, Vk)
    return out.reshape(n, h, d)


def phase2_rows_one_head(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                         positions: Sequence[int], scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dense phase-2 outputs and lse of sampled query rows for one kv head.

    ``q_rows``: ``[n, h, d]`` at absolute positions ``positions``; ``K``, ``V``:
    ``[N, d]`` the whole cache of the kv head (context then tail). Query at
    position p sees rows ``[0, p]``. Returns ``(O [n, h, d], lse [n, h])``.
    """
    n, h, d = q_rows.shape
    O = np.zeros((n, h, d), dtype=np.float64)
    LSE = np.zeros((n, h), dtype=np.float64)
    for k, p in enumerate(positions):
        Kk = np.asarray(K[:p + 1], dtype=np.float64)
        Vk = np.asarray(V[:p + 1], dtype=np.float64)
        S = scale * (np.asarray(q_rows[k], dtype=np.float64) @ Kk.T)
        O[k], LSE[k] = _softmax_rows(S, Vk)
    return O, LSE


# --------------------------------------------------------------------------
# Brute force on tiny inputs: scalar loops, math.exp and math.fsum
# --------------------------------------------------------------------------

def _bf_attend(q, keys_k, keys_v, scale):
    s = [scale * math.fsum(qi * ki for qi, ki in zip(q, k)) for k in keys_k]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    d = len(keys_v[0])
    o = [math.fsum(e[r] * keys_v[r][c] for r in range(len(e))) / z for c in range(d)]
    return o, m + math.log(z)


def brute_force_phase1(q_ctx, k_ctx, v_ctx, block_len, anchor_len, scale):
    """Scalar-loop phase 1 over nested lists / arrays; returns nested lists."""
    B, L, Hq = len(q_ctx), len(q_ctx[0]), len(q_ctx[0][0])
    Hkv = len(k_ctx[0][0])
    G = Hq // Hkv
    out = []
    for s in range(B):
        rows_out = []
        for r in range(L):
            i = r // block_len
            keys = ([j for j in range(anchor_len)] if i > 0 else []) + \
                   [j for j in range(i * block_len, r + 1)]
            heads = []
            for h in range(Hq):
                g = h // G
                o, _ = _bf_attend(q_ctx[s][r][h], [k_ctx[s][j][g] for j in keys],
                                  [v_ctx[s][j][g] for j in keys], scale)
                heads.append(o)
            rows_out.append(heads)
        out.append(rows_out)
    return out


def brute_force_phase2(q_rows, k_all, v_all, positions, scale):
    """Scalar-loop dense phase 2; returns (outputs, lse) as nested lists."""
    B, Hq = len(q_rows), len(q_rows[0][0])
    Hkv = len(k_all[0][0])
    G = Hq // Hkv
    O, LSE = [], []
    for s in range(B):
        orow, lrow = [], []
        for j, p in enumerate(positions):
            oh, lh = [], []
            for h in range(Hq):
                g = h // G
                o, l = _bf_attend(q_rows[s][j][h], [k_all[s][r][g] for r in range(p + 1)],
                                  [v_all[s][r][g] for r in range(p + 1)], scale)
                oh.append(o)
                lh.append(l)
            orow.append(oh)
            lrow.append(lh)
        O.append(orow)
        LSE.append(lrow)
    return O, LSE


# --------------------------------------------------------------------------
# Rotary position embedding in phase 1: the anchor's position ids
# --------------------------------------------------------------------------
#
# paperhub.cn rebuttal, reply to reviewer x5MA point 1: with the first block
# as the anchor, the position ids given to the anchor tokens during the local
# attention of phase 1 change the result little. The pages name no
# positional scheme and give no formula. Readings:
#   * rotary position embedding (RoFormer), the scheme of the Llama models
#     the pages evaluate, with half-split pairing: element i of a head vector
#     is rotated together with element i + d/2 (i < d/2) by the angle whose
#     cosine and sine are entry [pos][i] of caller-given tables;
#   * two anchor modes for a row of block i >= 1:
#       ORIGINAL - anchor row j keeps position j (its place in the context);
#       ADJACENT - anchor row j takes position i*b - a + j, directly before
#                  the block, as if the anchor had been prepended to it;
#     every other key and every query keeps its context position.
ROPE_ORIGINAL, ROPE_ADJACENT = 0, 1


def rope_rotate(x: np.ndarray, cos_rows: np.ndarray, sin_rows: np.ndarray) -> np.ndarray:
    """Rotate head vectors ``x[..., d]`` by the table rows ``cos_rows[..., d/2]``,
    ``sin_rows[..., d/2]`` (one row per vector), in float64:
    ``y_i = x_i c_i - x_{i+d/2} s_i``, ``y_{i+d/2} = x_{i+d/2} c_i + x_i s_i``."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos_rows, dtype=np.float64)
    s = np.asarray(sin_rows, dtype=np.float64)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def _round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def rope_rotate_f32(x: np.ndarray, cos_rows: np.ndarray, sin_rows: np.ndarray) -> np.ndarray:
    """The rotation in float32 arithmetic, every product and the sum or
    difference rounded to float32 on its own (no fused multiply-add): the
    rotated keys of an fp32 model. Returns float32."""
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    c = np.asarray(cos_rows, dtype=np.float32)
    s = np.asarray(sin_rows, dtype=np.float32)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([(lo * c) - (hi * s), (hi * c) + (lo * s)], axis=-1).astype(np.float32)


def rope_rotate_bf16(x: np.ndarray, cos_rows: np.ndarray, sin_rows: np.ndarray) -> np.ndarray:
    """The rotation as a bf16 model stores its rotated keys: the float32 form
    above, then rounded to bfloat16. Returns float64 values."""
    return _round_bf16(rope_rotate_f32(x, cos_rows, sin_rows)).astype(np.float64)


def phase1_rope_positions(block_len: int, anchor_len: int, i: int, mode: int) -> np.ndarray:
    """Position ids of the anchor rows ``[0, a)`` as block ``i >= 1`` sees them."""
    j = np.arange(anchor_len, dtype=np.int64)
    return j if mode == ROPE_ORIGINAL else i * block_len - anchor_len + j


def phase1_rope(q_ctx: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, block_len: int,
                anchor_len: int, scale: float, cos_tab: np.ndarray, sin_tab: np.ndarray,
                mode: int) -> np.ndarray:
    """Phase 1 with rotary position embedding: ``q_ctx`` and ``k_ctx`` hold the
    un-rotated head vectors ``[B, L, H, d]``; every query and key is rotated
    at its position id (context position; anchor rows per ``mode``) before
    the same blockwise-local causal attention as ``phase1``. float64, exact
    rotations."""
    B, L, Hq, d = q_ctx.shape
    Hkv = k_ctx.shape[2]
    out = np.zeros((B, L, Hq, d), dtype=np.float64)
    n_blocks = -(-L // block_len)
    ctx_pos = np.arange(L, dtype=np.int64)
    for s in range(B):
        for i in range(n_blocks):
            lo, hi = i * block_len, min((i + 1) * block_len, L)
            n_loc = hi - lo
            if i > 0:
                anc_rows = np.arange(anchor_len, dtype=np.int64)
                anc_pos = phase1_rope_positions(block_len, anchor_len, i, mode)
            else:
                anc_rows = anc_pos = np.arange(0, dtype=np.int64)
            rows = np.concatenate([anc_rows, np.arange(lo, hi)])
            pos = np.concatenate([anc_pos, ctx_pos[lo:hi]])
            visible = np.zeros((n_loc, rows.size), dtype=bool)
            visible[:, :anc_rows.size] = True
            visible[:, anc_rows.size:] = np.tri(n_loc, dtype=bool)  # causal, diagonal included
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                Q = rope_rotate(q_ctx[s, lo:hi, h], cos_tab[lo:hi], sin_tab[lo:hi])
                K = rope_rotate(k_ctx[s, rows, g], cos_tab[pos], sin_tab[pos])
                V = v_ctx[s, rows, g]
                S = np.where(visible, (Q @ K.T) * scale, -np.inf)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                out[s, lo:hi, h] = (E @ V) / np.sum(E, axis=1, keepdims=True)
    return out


def phase1_rope_rows_one_head(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                              rows: Sequence[int], block_len: int, anchor_len: int,
                              scale: float, cos_tab: np.ndarray, sin_tab: np.ndarray,
                              mode: int) -> np.ndarray:
    """``phase1_rope`` for sampled context rows of the query heads of one kv
    head (arguments as ``phase1_rows_one_head``, inputs not yet rotated):
    each key is rotated at its position id (anchor rows per ``mode``), each
    query at its row. Returns ``[n, h, d]``."""
    out = np.zeros(q_rows.shape, dtype=np.float64)
    for k, r in enumerate(rows):
        r = int(r)
        i = r // block_len
        keys = phase1_key_rows(r, block_len, anchor_len)
        n_anc = anchor_len if i > 0 else 0
        pos = keys.copy()
        if n_anc:
            pos[:n_anc] = phase1_rope_positions(block_len, anchor_len, i, mode)
        Kk = rope_rotate(np.asarray(K[keys], dtype=np.float64), cos_tab[pos], sin_tab[pos])
        Qr = rope_rotate(np.asarray(q_rows[k], dtype=np.float64), cos_tab[r], sin_tab[r])
        S = scale * (Qr @ Kk.T)
        out[k], _ = _softmax_rows(S, np.asarray(V[keys], dtype=np.float64))
    return out
