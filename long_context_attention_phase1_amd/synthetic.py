"""Seeded synthetic inputs for the Star Attention hot path.

This module only draws numbers and lays them out; it contains none of the
attention arithmetic. Both the GPU path (through the tests and the bench) and
the CPU oracle take their inputs from here, so the two sides always see the
exact same bf16 / fp32 values.

Workloads follow the pages' long-context setting (Star Attention, PMLR page,
Abstract: context processed in blocks, then query and response tokens; the
paperhub.cn rebuttal, reply to reviewer dnhh point 3: a 128K context cut into
32K blocks with a 32K anchor, and reply to EMsM point 4: fixed 32K blocks up
to 1M tokens). The head layout is the Llama-3.1-8B / 70B attention shape.

Stream layout (seekable): every tensor is cut into chunks of ``CHUNK`` tokens;
chunk ``c`` of tensor ``t`` for sequence ``s`` is drawn from its own PCG64
stream seeded with ``SeedSequence([seed, t, s, c])`` as float32 standard
normals in ``[token][head][dim]`` order. bf16 values are the float32 samples
rounded to nearest-even. Any row can therefore be regenerated on its own.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

CHUNK = 4096

# tensor ids of the seekable stream
T_QCTX, T_K, T_V, T_QTAIL, T_KTAIL, T_VTAIL, T_PEAK = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer workload (sizes only; no arithmetic)."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    block_len: int
    anchor_len: int
    n_query: int          # query tokens (phase 2, one call)
    n_decode: int         # decode steps (phase 2, one token each)
    dtype: str            # "bf16" or "f32"
    peak_frac: float = 0.0    # fraction of context K rows scaled up
    peak_factor: float = 1.0  # the scale applied to those rows
    seed: int = 0

    @property
    def n_blocks(self) -> int:
        return -(-self.ctx_len // self.block_len)

    @property
    def tail_cap(self) -> int:
        return self.n_query + self.n_decode

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the hot-path scope table.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 1, 64, 512, 128, 128, 16, 8, "f32"),
    "llama8b_32k": Workload("llama8b_32k", 1, 32, 8, 128, 32768, 4096, 4096,
                            64, 128, "bf16"),
    "llama8b_128k_peaked": Workload("llama8b_128k_peaked", 1, 32, 8, 128,
                                    131072, 16384, 16384, 64, 256, "bf16",
                                    peak_frac=0.01, peak_factor=8.0),
    "llama8b_1m": Workload("llama8b_1m", 1, 32, 8, 128, 1048576, 32768,
                           32768, 32, 64, "bf16"),
    "llama70b_256k_b4": Workload("llama70b_256k_b4", 4, 64, 8, 128, 262144,
                                 32768, 32768, 128, 128, "bf16"),
}

# Variants of the 128K workload that the pages discuss, as performance
# sweeps (same heads, inputs and peaked rows; 64 decode steps): the block
# fractions L/4, L/16 and L/32 beside the L/8 of the 128K workload (paperhub.cn
# review page, reply to reviewer x5MA point 3), an anchor shorter than the
# block (reply to EMsM point 5: the anchor is at most one block), and a
# context that is a multiple of neither the block nor the 64-row cache tile
# (ragged last block, unaligned edges).
_C3 = WORKLOADS["llama8b_128k_peaked"]
SWEEPS: Dict[str, Workload] = {
    "sweep_128k_b32k": _C3.replace(name="sweep_128k_b32k", block_len=32768, anchor_len=32768,
                                   n_decode=64),
    "sweep_128k_b8k": _C3.replace(name="sweep_128k_b8k", block_len=8192, anchor_len=8192,
                                  n_decode=64),
    "sweep_128k_b4k": _C3.replace(name="sweep_128k_b4k", block_len=4096, anchor_len=4096,
                                  n_decode=64),
    "sweep_128k_a4k_b16k": _C3.replace(name="sweep_128k_a4k_b16k", anchor_len=4096,
                                       n_decode=64),
    "sweep_125k_ragged": _C3.replace(name="sweep_125k_ragged", ctx_len=125003, n_decode=64),
}


def rope_tables(head_dim: int, n_pos: int, theta: float = 500000.0):
    """Rotary-embedding tables of a model (input data, like its weights):
    float32 ``cos``, ``sin`` of shape ``[n_pos, head_dim / 2]`` with angle
    ``pos * theta ** (-2 i / head_dim)``, computed in float64. The default
    base is the Llama-3 models' one."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / head_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def workload(name: str) -> Workload:
    """A workload of the scope table or a sweep variant, by name."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in SWEEPS:
        return SWEEPS[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS) + sorted(SWEEPS)}")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns the uint16 bit patterns.

    NaN never occurs in these inputs (finite normals times powers of two).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _chunk_normals(seed: int, tensor: int, seq: int, chunk: int, n: int) -> np.ndarray:
    ss = np.random.SeedSequence([seed, tensor, seq, chunk])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(n, dtype=np.float32)


def peaked_rows(w: Workload, seq: int) -> np.ndarray:
    """Context token indices whose K rows are scaled by ``peak_factor``.

    Per (sequence, kv head): ``round(peak_frac * ctx_len)`` distinct token
    indices. Returns an int64 array ``[n_kv_heads, n_peak]`` (sorted rows).
    """
    n_peak = int(round(w.peak_frac * w.ctx_len))
    out = np.zeros((w.n_kv_heads, n_peak), dtype=np.int64)
    if n_peak == 0:
        return out
    for g in range(w.n_kv_heads):
        ss = np.random.SeedSequence([w.seed, T_PEAK, seq, g])
        rng = np.random.Generator(np.random.PCG64(ss))
        out[g] = np.sort(rng.choice(w.ctx_len, size=n_peak, replace=False))
    return out


def _rows_f32(w: Workload, tensor: int, seq: int, tok0: int, tok1: int,
              n_heads: int) -> np.ndarray:
    """float32 samples of rows [tok0, tok1) of one tensor: [n, n_heads, d]."""
    d = w.head_dim
    per_tok = n_heads * d
    out = np.empty((max(tok1 - tok0, 0), n_heads, d), dtype=np.float32)
    if tok1 <= tok0:
        return out
    for c in range(tok0 // CHUNK, (tok1 - 1) // CHUNK + 1):
        a, b = c * CHUNK, (c + 1) * CHUNK
        x = _chunk_normals(w.seed, tensor, seq, c, CHUNK * per_tok).reshape(CHUNK, n_heads, d)
        lo, hi = max(a, tok0), min(b, tok1)
        out[lo - tok0:hi - tok0] = x[lo - a:hi - a]
    return out


def rows(w: Workload, tensor: int, seq: int, tok0: int, tok1: int) -> np.ndarray:
    """Rows [tok0, tok1) of one input tensor for one sequence.

    Returns ``[n, H, d]``: uint16 bf16 bit patterns for bf16 workloads,
    float32 values for f32 workloads. ``tensor`` is one of the ``T_*`` ids;
    context tensors take token indices in ``[0, ctx_len)``, tail tensors in
    ``[0, n_query + n_decode)``.
    """
    n_heads = w.n_q_heads if tensor in (T_QCTX, T_QTAIL) else w.n_kv_heads
    x = _rows_f32(w, tensor, seq, tok0, tok1, n_heads)
    if tensor == T_K and w.peak_frac > 0.0:
        pk = peaked_rows(w, seq)
        for g in range(w.n_kv_heads):
            sel = pk[g][(pk[g] >= tok0) & (pk[g] < tok1)] - tok0
            x[sel, g, :] *= np.float32(w.peak_factor)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of generator output as float64 (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def full_tensor(w: Workload, tensor: int, threads: Optional[int] = None) -> np.ndarray:
    """Whole tensor ``[B, T, H, d]`` (bf16 bits or float32), chunks drawn in parallel."""
    ctx = tensor in (T_QCTX, T_K, T_V)
    n_tok = w.ctx_len if ctx else w.tail_cap
    n_heads = w.n_q_heads if tensor in (T_QCTX, T_QTAIL) else w.n_kv_heads
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.empty((w.batch, n_tok, n_heads, w.head_dim), dtype=dt)
    jobs = [(s, c * CHUNK, min((c + 1) * CHUNK, n_tok))
            for s in range(w.batch) for c in range(-(-n_tok // CHUNK))]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))

    def one(job):
        s, a, b = job
        out[s, a:b] = rows(w, tensor, s, a, b)

    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            one(j)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, jobs))
    return out


def make_inputs(w: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of a workload, token-major ``[B, T, H, d]``.

    Keys: ``q_ctx``, ``k_ctx``, ``v_ctx`` (context, T = ctx_len) and
    ``q_tail``, ``k_tail``, ``v_tail`` (T = n_query + n_decode: the query
    tokens followed by the pre-drawn decode tokens).
    """
    ids = {"q_ctx": T_QCTX, "k_ctx": T_K, "v_ctx": T_V,
           "q_tail": T_QTAIL, "k_tail": T_KTAIL, "v_tail": T_VTAIL}
    return {k: full_tensor(w, t, threads) for k, t in ids.items()}
