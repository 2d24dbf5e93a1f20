"""Planted mistakes in a copy of the oracle must each trip at least one pin.

Every mutant is built on the CPU from the oracle's source text with a single
textual edit (a dropped term, an off-by-one, a wrong index or sign, a wrong
log base, a missing normalisation), loaded as a throwaway module, and run
through every pin of ``oracle_pins``. The real oracle is never modified.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "star_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("causal_excludes_diagonal_row_fn",
     "local = np.arange(i * block_len, r + 1, dtype=np.int64)",
     "local = np.arange(i * block_len, r, dtype=np.int64)"),
    ("causal_sees_one_future_key",
     "np.tril(np.ones((n_loc, n_loc), dtype=bool))",
     "np.tril(np.ones((n_loc, n_loc), dtype=bool), 1)"),
    ("anchor_dropped",
     "anc = np.arange(anchor_len) if i > 0 else np.arange(0)",
     "anc = np.arange(0)"),
    ("anchor_also_on_block0",
     "anc = np.arange(anchor_len) if i > 0 else np.arange(0)",
     "anc = np.arange(anchor_len)"),
    ("anchor_off_by_one",
     "anc = np.arange(anchor_len) if i > 0 else np.arange(0)",
     "anc = np.arange(anchor_len - 1) if i > 0 else np.arange(0)"),
    ("row_fn_anchor_on_block0",
     "    if i == 0:\n        return local\n",
     "    if i < 0:\n        return local\n"),
    ("gqa_modulo_mapping",
     "return h // (n_q_heads // n_kv_heads)",
     "return h % n_kv_heads"),
    ("scale_without_sqrt",
     "1.0 / math.sqrt(head_dim) if softmax_scale",
     "1.0 / head_dim if softmax_scale"),
    ("scale_ignores_override",
     "if softmax_scale == 0.0 else float(softmax_scale)",
     "if softmax_scale == 0.0 else 1.0"),
    ("lse_log2",
     "return (e @ V) / z, m + math.log(z)",
     "return (e @ V) / z, m + math.log2(z)"),
    ("lse_drops_max",
     "return (e @ V) / z, m + math.log(z)",
     "return (e @ V) / z, math.log(z)"),
    ("attend_unnormalised",
     "return (e @ V) / z, m + math.log(z)",
     "return (e @ V), m + math.log(z)"),
    ("phase1_normalised_by_total",
     "out[s, lo:hi, h] = (E @ V) / E.sum(axis=1, keepdims=True)",
     "out[s, lo:hi, h] = (E @ V) / E.sum()"),
    ("phase1_transposed_scores",
     "S = scale * (Q @ K.T)",
     "S = scale * (Q @ K.T).T[:Q.shape[0], :K.shape[0]] if Q.shape[0] == K.shape[0] else scale * (Q @ K.T)"),
    ("phase1_missing_scale",
     "S = scale * (Q @ K.T)",
     "S = (Q @ K.T)"),
    ("merge_weight_sign",
     "w = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m), 0.0)",
     "w = np.where(finite, np.exp(m - np.where(finite, lse_parts, 0.0)), 0.0)"),
    ("merge_unnormalised",
     "o = (w @ o_parts) / z",
     "o = (w @ o_parts)"),
    ("merge_lse_drops_max",
     "    o = (w @ o_parts) / z\n    return o, m + math.log(z)",
     "    o = (w @ o_parts) / z\n    return o, math.log(z)"),
    ("partial_sees_future",
     "top = min(hi, pos + 1)",
     "top = hi"),
    ("partial_excludes_self",
     "top = min(hi, pos + 1)",
     "top = min(hi, pos)"),
    ("pieces_overlap_tail",
     "pieces = [(lo, min(lo + block_len, ctx_len)) for lo in range(0, ctx_len, block_len)]",
     "pieces = [(lo, lo + block_len) for lo in range(0, ctx_len, block_len)]"),
    ("pieces_drop_tail",
     "    if kv_len > ctx_len:\n        pieces.append((ctx_len, kv_len))\n",
     "    if kv_len < ctx_len:\n        pieces.append((ctx_len, kv_len))\n"),
    ("dense_excludes_self",
     "k_all[s, :p + 1, g], v_all[s, :p + 1, g], scale)\n                O[s, j, h], LSE[s, j, h] = o, l",
     "k_all[s, :p, g], v_all[s, :p, g], scale)\n                O[s, j, h], LSE[s, j, h] = o, l"),
    ("dense_v_from_k",
     "k_all[s, :p + 1, g], v_all[s, :p + 1, g], scale)\n                O[s, j, h], LSE[s, j, h] = o, l",
     "k_all[s, :p + 1, g], k_all[s, :p + 1, g], scale)\n                O[s, j, h], LSE[s, j, h] = o, l"),
    ("decode_excludes_self",
     "kv_len = L + t + 1",
     "kv_len = L + t"),
    ("decode_query_step_sees_all_tail",
     "[L + j for j in range(n_query)], scale)",
     "[L + n_query - 1 for j in range(n_query)], scale)"),
    ("block_rows_see_own_future",
     "visible[:, len(anc):] = blk[None, :] <= rows[:, None]",
     "visible[:, len(anc):] = blk[None, :] <= rows[:, None] + 1"),
    ("block_rows_anchor_on_block0",
     "anc = np.arange(anchor_len if i > 0 else 0, dtype=np.int64)",
     "anc = np.arange(anchor_len, dtype=np.int64)"),
    ("sampled_p1_no_anchor",
     "keys = phase1_key_rows(int(r), block_len, anchor_len)",
     "keys = phase1_key_rows(int(r), block_len, 0)[anchor_len * 0:] if r < block_len else np.arange(r // block_len * block_len, r + 1)"),
    ("sampled_p2_excludes_self",
     "Kk = np.asarray(K[:p + 1], dtype=np.float64)\n        Vk = np.asarray(V[:p + 1], dtype=np.float64)",
     "Kk = np.asarray(K[:p], dtype=np.float64)\n        Vk = np.asarray(V[:p], dtype=np.float64)"),
    ("sampled_softmax_lse_log2",
     "return (E @ V) / z, (m + np.log(z))[:, 0]",
     "return (E @ V) / z, (m + np.log2(z))[:, 0]"),
    ("sampled_softmax_unnormalised",
     "return (E @ V) / z, (m + np.log(z))[:, 0]",
     "return (E @ V), (m + np.log(z))[:, 0]"),
    ("rope_sine_sign",
     "return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)",
     "return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)"),
    ("rope_pairs_neighbours",
     "    lo, hi = x[..., :h], x[..., h:]\n    return np.concatenate([lo * c - hi * s",
     "    lo, hi = x[..., 0::2], x[..., 1::2]\n    return np.concatenate([lo * c - hi * s"),
    ("rope_bf16_rounds_half_up",
     "u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16",
     "u = (u + 0x8000) >> 16 << 16"),
    ("rope_bf16_fused_in_float64",
     "return np.concatenate([(lo * c) - (hi * s), (hi * c) + (lo * s)], axis=-1).astype(np.float32)",
     "return np.concatenate([(lo.astype(np.float64) * c) - (hi.astype(np.float64) * s), (hi.astype(np.float64) * c) + (lo.astype(np.float64) * s)], axis=-1).astype(np.float32)"),
    ("rope_adjacent_no_anchor_shift",
     "return j if mode == ROPE_ORIGINAL else i * block_len - anchor_len + j",
     "return j if mode == ROPE_ORIGINAL else i * block_len + j"),
    ("rope_adjacent_ignored",
     "return j if mode == ROPE_ORIGINAL else i * block_len - anchor_len + j",
     "return j"),
    ("rope_query_not_rotated",
     "Q = rope_rotate(q_ctx[s, lo:hi, h], cos_tab[lo:hi], sin_tab[lo:hi])",
     "Q = q_ctx[s, lo:hi, h]"),
    ("rope_keys_at_row_not_position",
     "K = rope_rotate(k_ctx[s, rows, g], cos_tab[pos], sin_tab[pos])",
     "K = rope_rotate(k_ctx[s, rows, g], cos_tab[rows], sin_tab[rows])"),
    ("rope_phase1_sees_one_future_key",
     "visible[:, anc_rows.size:] = np.tri(n_loc, dtype=bool)",
     "visible[:, anc_rows.size:] = np.tri(n_loc, k=1, dtype=bool)"),
    ("rope_phase1_missing_scale",
     "S = np.where(visible, (Q @ K.T) * scale, -np.inf)",
     "S = np.where(visible, (Q @ K.T), -np.inf)"),
    ("rope_phase1_normalised_by_total",
     "out[s, lo:hi, h] = (E @ V) / np.sum(E, axis=1, keepdims=True)",
     "out[s, lo:hi, h] = (E @ V) / np.sum(E)"),
    ("rope_rows_anchor_at_original_ids",
     "            pos[:n_anc] = phase1_rope_positions(block_len, anchor_len, i, mode)",
     "            pos[:n_anc] = phase1_rope_positions(block_len, anchor_len, i, ROPE_ORIGINAL)"),
    ("rope_rows_query_at_block_start",
     "Qr = rope_rotate(np.asarray(q_rows[k], dtype=np.float64), cos_tab[r], sin_tab[r])",
     "Qr = rope_rotate(np.asarray(q_rows[k], dtype=np.float64), cos_tab[i * block_len], sin_tab[i * block_len])"),
    ("rope_phase1_anchor_on_block0",
     "            if i > 0:\n                anc_rows = np.arange(anchor_len, dtype=np.int64)",
     "            if i >= 0:\n                anc_rows = np.arange(anchor_len, dtype=np.int64)"),
]


def _load_mutant(name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation {name}: pattern occurs {text.count(old)} times"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(name, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin catches mutant {name}"
