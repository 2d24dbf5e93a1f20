"""A synthetic workload resident on the GPU, driven through the C ABI.

``Pipeline`` holds one workload's inputs, KV cache and outputs in device
memory and runs each step of the path as one call of libstarattn through
the Python binding: the context KV write, phase 1, the query step and the
decode steps. It only allocates device tensors and marshals arguments;
every arithmetic step runs in the HIP kernels. The bench, the smoke check
and the GPU tests all drive the path through it.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as sa
from . import synthetic as syn

NAN_BF16 = 0x7FC0


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Pipeline:
    """One workload resident on the GPU: inputs, KV cache, outputs."""

    def __init__(self, w: syn.Workload, inputs=None, device="cuda", fill_nan=True, threads=None):
        self.w = w
        self.dtype = sa.STAR_BF16 if w.dtype == "bf16" else sa.STAR_F32
        self.desc = sa.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_len,
                                 w.block_len, w.anchor_len, w.tail_cap, self.dtype)
        self.inputs = inputs if inputs is not None else syn.make_inputs(w, threads)
        self.dev = {k: to_device(v, w.dtype, device) for k, v in self.inputs.items()}
        self.k_cache = sa.alloc_kv_cache(self.desc, device)
        self.v_cache = sa.alloc_kv_cache(self.desc, device)
        if fill_nan:  # unwritten cache rows read as NaN, so a stray read shows up
            for c in (self.k_cache, self.v_cache):
                if w.dtype == "bf16":
                    c.view(torch.int16).fill_(NAN_BF16)
                else:
                    c.fill_(float("nan"))
        elt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.elt = elt
        self.o_ctx = torch.empty(w.batch, w.ctx_len, w.n_q_heads, w.head_dim, dtype=elt,
                                 device=device)
        # per-row tail slices, contiguous
        self.q_tail_rows = [self.dev["q_tail"][:, t:t + 1].contiguous() for t in range(w.tail_cap)]
        self.k_tail_rows = [self.dev["k_tail"][:, t:t + 1].contiguous() for t in range(w.tail_cap)]
        self.v_tail_rows = [self.dev["v_tail"][:, t:t + 1].contiguous() for t in range(w.tail_cap)]
        self.q_query = self.dev["q_tail"][:, :w.n_query].contiguous()
        self.k_query = self.dev["k_tail"][:, :w.n_query].contiguous()
        self.v_query = self.dev["v_tail"][:, :w.n_query].contiguous()
        self._ws = {}

    # -- phase 1 -----------------------------------------------------------
    def write_context(self):
        w = self.w
        sa.star_kv_write(self.desc, self.k_cache, self.v_cache, 0, self.dev["k_ctx"],
                         self.dev["v_ctx"], w.ctx_len)

    def phase1(self):
        sa.star_attn_phase1(self.desc, self.k_cache, self.v_cache, self.dev["q_ctx"], self.o_ctx)
        return self.o_ctx

    # -- phase 2 -----------------------------------------------------------
    def workspace(self, kv_len, n_query):
        n_split = sa.star_attn_phase2_plan(self.desc, kv_len, n_query)
        key = (n_query, n_split)
        if key not in self._ws:
            w = self.w
            o_part = torch.empty(w.batch, n_query, w.n_q_heads, n_split, w.head_dim,
                                 dtype=torch.float32, device=self.o_ctx.device)
            lse_part = torch.empty(w.batch, n_query, w.n_q_heads, n_split, dtype=torch.float32,
                                   device=self.o_ctx.device)
            o = torch.empty(w.batch, n_query, w.n_q_heads, w.head_dim, dtype=self.elt,
                            device=self.o_ctx.device)
            lse = torch.empty(w.batch, n_query, w.n_q_heads, dtype=torch.float32,
                              device=self.o_ctx.device)
            self._ws[key] = (n_split, o_part, lse_part, o, lse)
        return self._ws[key]

    # -- rotary embedding (phase 1) ------------------------------------------
    def rope(self, mode, theta=500000.0):
        """Device rotary tables for every cache row and a star_rope over them."""
        w = self.w
        c, s_ = syn.rope_tables(w.head_dim, w.ctx_len + w.tail_cap, theta)
        self.rope_host = (c, s_)
        self._rope_dev = (torch.from_numpy(c).to(self.o_ctx.device),
                          torch.from_numpy(s_).to(self.o_ctx.device))
        return sa.make_rope(self._rope_dev[0], self._rope_dev[1], mode)

    def write_context_rope(self, rope):
        w = self.w
        sa.star_kv_write_rope(self.desc, self.k_cache, self.v_cache, 0, self.dev["k_ctx"],
                              self.dev["v_ctx"], w.ctx_len, rope)

    def phase1_rope(self, rope):
        sa.star_attn_phase1_rope(self.desc, self.k_cache, self.v_cache, self.dev["q_ctx"], rope,
                                 self.o_ctx)
        return self.o_ctx

    # the phase-2 calls on the cache (the paged pipeline overrides these three)
    def kv_write2(self, pos0, k, v, n_tok):
        sa.star_kv_write(self.desc, self.k_cache, self.v_cache, pos0, k, v, n_tok)

    def partial2(self, kv_len, q, n_query, o_part, lse_part):
        sa.star_attn_phase2_partial(self.desc, self.k_cache, self.v_cache, kv_len, q, n_query,
                                    o_part, lse_part)

    def decode_call(self, kv_len, row, o_part, lse_part, o, lse):
        """star_attn_decode_step for tail row ``row`` at kv_len."""
        sa.star_attn_decode_step(self.desc, self.k_cache, self.v_cache, kv_len,
                                 self.q_tail_rows[row], self.k_tail_rows[row],
                                 self.v_tail_rows[row], 1, o_part, lse_part, o, self.dtype, lse)

    def attend(self, kv_len, q, n_query):
        n_split, o_part, lse_part, o, lse = self.workspace(kv_len, n_query)
        self.partial2(kv_len, q, n_query, o_part, lse_part)
        sa.star_attn_lse_merge(self.desc, n_query, n_split, o_part, lse_part, o, self.dtype, lse)
        return o, lse

    def query_step(self):
        """The query step as one call: append the n_query rows' K/V, the
        partials and the merge (star_attn_decode_step[_paged] for n_query
        rows)."""
        w = self.w
        kv_len = w.ctx_len + w.n_query
        n_split, o_part, lse_part, o, lse = self.workspace(kv_len, w.n_query)
        self.step_call(kv_len, self.q_query, self.k_query, self.v_query, w.n_query, o_part,
                       lse_part, o, lse)
        return o, lse

    def query_step_separate(self):
        """The query step as three calls: kv_write, partials, merge."""
        w = self.w
        self.kv_write2(w.ctx_len, self.k_query, self.v_query, w.n_query)
        return self.attend(w.ctx_len + w.n_query, self.q_query, w.n_query)

    def step_call(self, kv_len, q, k, v, n_query, o_part, lse_part, o, lse):
        """star_attn_decode_step for n_query rows ending at kv_len."""
        sa.star_attn_decode_step(self.desc, self.k_cache, self.v_cache, kv_len, q, k, v, n_query,
                                 o_part, lse_part, o, self.dtype, lse)

    def decode_step(self, t):
        """Decode step t (0-based): append tail row n_query + t, attend with it."""
        w = self.w
        row = w.n_query + t
        self.kv_write2(w.ctx_len + row, self.k_tail_rows[row], self.v_tail_rows[row], 1)
        return self.attend(w.ctx_len + row + 1, self.q_tail_rows[row], 1)

    def decode_step_fused(self, t):
        """Decode step t through star_attn_decode_step (append + partials + merge)."""
        w = self.w
        row = w.n_query + t
        kv_len = w.ctx_len + row + 1
        n_split, o_part, lse_part, o, lse = self.workspace(kv_len, 1)
        self.decode_call(kv_len, row, o_part, lse_part, o, lse)
        return o, lse

    def run_tail(self, fused=False):
        """Query step then every decode step; returns host arrays [B, T, Hq, d], [B, T, Hq].
        fused: each step as one star_attn_decode_step call; else as the
        separate kv_write, partial and merge calls."""
        w = self.w
        o, lse = self.query_step() if fused else self.query_step_separate()
        outs, lses = [to_host_f64(o)], [lse.cpu().numpy().astype(np.float64)]
        for t in range(w.n_decode):
            o, lse = self.decode_step_fused(t) if fused else self.decode_step(t)
            outs.append(to_host_f64(o))
            lses.append(lse.cpu().numpy().astype(np.float64))
        return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)


class PagedPipeline(Pipeline):
    """The same workload with phase 2 on a paged cache: page pools with
    ``spare`` extra pages, a block table that is a seeded random permutation
    of the pages, unused pages NaN-filled (a stray read shows up). Phase 1
    reads the contiguous cache, which ``write_context`` fills as well."""

    def __init__(self, w: syn.Workload, inputs=None, device="cuda", fill_nan=True, threads=None,
                 spare=5, table_seed=7):
        super().__init__(w, inputs=inputs, device=device, fill_nan=fill_nan, threads=threads)
        self.maxp = -(-(w.ctx_len + w.tail_cap) // sa.STAR_KV_TILE)
        self.n_pages = w.batch * self.maxp + spare
        self.k_pages = sa.alloc_kv_pages(self.desc, self.n_pages, device)
        self.v_pages = sa.alloc_kv_pages(self.desc, self.n_pages, device)
        for c in (self.k_pages, self.v_pages):
            if w.dtype == "bf16":
                c.view(torch.int16).fill_(NAN_BF16)
            else:
                c.fill_(float("nan"))
        perm = np.random.default_rng(table_seed).permutation(self.n_pages)[: w.batch * self.maxp]
        self.table_host = perm.reshape(w.batch, self.maxp).astype(np.int32)
        self.table = torch.from_numpy(self.table_host).to(device)

    def write_context(self):
        super().write_context()
        w = self.w
        sa.star_kv_write_paged(self.desc, self.k_pages, self.v_pages, self.table, 0,
                               self.dev["k_ctx"], self.dev["v_ctx"], w.ctx_len)

    def kv_write2(self, pos0, k, v, n_tok):
        sa.star_kv_write_paged(self.desc, self.k_pages, self.v_pages, self.table, pos0, k, v, n_tok)

    def partial2(self, kv_len, q, n_query, o_part, lse_part):
        sa.star_attn_phase2_partial_paged(self.desc, self.k_pages, self.v_pages, self.table,
                                          kv_len, q, n_query, o_part, lse_part)

    def decode_call(self, kv_len, row, o_part, lse_part, o, lse):
        sa.star_attn_decode_step_paged(self.desc, self.k_pages, self.v_pages, self.table, kv_len,
                                       self.q_tail_rows[row], self.k_tail_rows[row],
                                       self.v_tail_rows[row], 1, o_part, lse_part, o, self.dtype,
                                       lse)

    def step_call(self, kv_len, q, k, v, n_query, o_part, lse_part, o, lse):
        sa.star_attn_decode_step_paged(self.desc, self.k_pages, self.v_pages, self.table, kv_len,
                                       q, k, v, n_query, o_part, lse_part, o, self.dtype, lse)
