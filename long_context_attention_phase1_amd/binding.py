"""ctypes binding of libstarattn (include/star_attn.h), same names as the C ABI.

Argument marshalling only: every step of the hot path runs in the HIP
kernels of ``libstarattn.so``. Tensor arguments are PyTorch device tensors
(device memory and streams are PyTorch's); their shapes, dtypes and
contiguity are checked here so that a wrong buffer raises instead of being
read out of bounds. Integer arguments are raw device pointers and are passed
as they are. The stream defaults to torch's current stream.

The library must be built (``python -m long_context_attention_phase1_amd.build``);
loading fails loudly otherwise, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstarattn.so")

STAR_OK = 0
STAR_ERR_INVALID_ARG = -1
STAR_ERR_SHAPE = -2
STAR_ERR_DTYPE = -3
STAR_ERR_UNSUPPORTED = -4
STAR_ERR_HIP = -5
STAR_BF16 = 0
STAR_F32 = 1
STAR_KV_TILE = 64

EXPORTS = ("star_kv_cache_bytes", "star_kv_write", "star_attn_phase1", "star_attn_phase2_plan",
           "star_attn_phase2_split_range", "star_attn_phase2_partial", "star_attn_lse_merge",
           "star_attn_decode_step", "star_attn_decode_step_noalloc", "star_kv_page_bytes", "star_kv_write_paged",
           "star_attn_phase2_partial_paged", "star_attn_decode_step_paged", "star_kv_write_rope",
           "star_attn_phase1_rope", "star_attn_strerror", "star_attn_abi_version")


class StarAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {star_attn_strerror(status)}")


class StarAttnDesc(ctypes.Structure):
    """Mirror of ``star_attn_desc``."""
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ctx_len", ctypes.c_int64), ("block_len", ctypes.c_int64),
                ("anchor_len", ctypes.c_int64), ("tail_cap", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class StarRope(ctypes.Structure):
    """Mirror of ``star_rope`` (device table pointers, rows, anchor mode)."""
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("n_pos", ctypes.c_int64),
                ("anchor_mode", ctypes.c_int32)]


STAR_ROPE_ORIGINAL = 0
STAR_ROPE_ADJACENT = 1

_lib = None


ABI_VERSION = 1  # STAR_ATTN_ABI_VERSION of include/star_attn.h that these signatures follow


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libstarattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m long_context_attention_phase1_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    D = ctypes.POINTER(StarAttnDesc)
    sig = {
        "star_kv_cache_bytes": (ctypes.c_size_t, [D]),
        "star_kv_write": (ctypes.c_int, [D, P, P, I64, P, P, I64, P]),
        "star_attn_phase1": (ctypes.c_int, [D, P, P, P, P, P]),
        "star_attn_phase2_plan": (ctypes.c_int, [D, I64, I64, ctypes.POINTER(I32)]),
        "star_attn_phase2_split_range": (ctypes.c_int, [D, I64, I64, I32, ctypes.POINTER(I64),
                                                        ctypes.POINTER(I64), ctypes.POINTER(I32)]),
        "star_attn_phase2_partial": (ctypes.c_int, [D, P, P, I64, P, I64, P, P, P]),
        "star_attn_lse_merge": (ctypes.c_int, [D, I64, I32, P, P, P, I32, P, P]),
        "star_attn_decode_step": (ctypes.c_int, [D, P, P, I64, P, P, P, I64, P, P, P, I32, P, P]),
        "star_attn_decode_step_noalloc": (ctypes.c_int, [D, P, P, I64, P, P, P, I64, P, I32, P, P]),
        "star_kv_page_bytes": (ctypes.c_size_t, [D]),
        "star_kv_write_rope": (ctypes.c_int, [D, P, P, I64, P, P, I64, ctypes.POINTER(StarRope), P]),
        "star_attn_phase1_rope": (ctypes.c_int, [D, P, P, P, ctypes.POINTER(StarRope), P, P]),
        "star_kv_write_paged": (ctypes.c_int, [D, P, P, P, I32, I64, P, P, I64, P]),
        "star_attn_phase2_partial_paged": (ctypes.c_int, [D, P, P, P, I32, I64, P, I64, P, P, P]),
        "star_attn_decode_step_paged": (ctypes.c_int, [D, P, P, P, I32, I64, P, P, P, I64, P, P, P,
                                                       I32, P, P]),
        "star_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "star_attn_abi_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if lib.star_attn_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.star_attn_abi_version()}, this binding "
                          f"marshals version {ABI_VERSION}: rebuild the library")
    _lib = lib
    return lib


def make_desc(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ctx_len: int,
              block_len: int, anchor_len: int, tail_cap: int, dtype: int = STAR_BF16,
              softmax_scale: float = 0.0) -> StarAttnDesc:
    return StarAttnDesc(batch, n_q_heads, n_kv_heads, head_dim, ctx_len, block_len, anchor_len,
                        tail_cap, dtype, softmax_scale)


# ---------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if not hasattr(stream, "cuda_stream") else stream.cuda_stream
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _elt(desc: StarAttnDesc):
    torch = _torch()
    return torch.bfloat16 if desc.dtype == STAR_BF16 else torch.float32


def _ptr(x, shape=None, dtype=None, name="buffer") -> Optional[int]:
    """Device pointer of a tensor (checked) or an integer passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an int pointer")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")
    return x.data_ptr()


def _cache_ptr(desc, x, name):
    if isinstance(x, int) or x is None:
        return x
    nbytes = star_kv_cache_bytes(desc)
    if x.numel() * x.element_size() < nbytes:
        raise ValueError(f"{name}: {x.numel() * x.element_size()} bytes < {nbytes}")
    return _ptr(x, name=name)


def _check(status: int, where: str):
    if status != STAR_OK:
        raise StarAttnError(status, where)


# ---------------------------------------------------------------- entry points

def star_attn_strerror(status: int) -> str:
    return load_library().star_attn_strerror(status).decode()


def star_attn_abi_version() -> int:
    return load_library().star_attn_abi_version()


def star_kv_cache_bytes(desc: StarAttnDesc) -> int:
    return load_library().star_kv_cache_bytes(ctypes.byref(desc))


def alloc_kv_cache(desc: StarAttnDesc, device="cuda"):
    """One K or V cache buffer (torch.empty of star_kv_cache_bytes)."""
    torch = _torch()
    nbytes = star_kv_cache_bytes(desc)
    if nbytes == 0:
        raise StarAttnError(STAR_ERR_INVALID_ARG, "alloc_kv_cache")
    elt = _elt(desc)
    return torch.empty(nbytes // torch.tensor([], dtype=elt).element_size(), dtype=elt,
                       device=device)


def star_kv_write(desc, k_cache, v_cache, pos0: int, k_src, v_src, n_tok: int, stream=None):
    shp = (desc.batch, n_tok, desc.n_kv_heads, desc.head_dim)
    elt = None if isinstance(k_src, int) else _elt(desc)
    st = load_library().star_kv_write(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        pos0, _ptr(k_src, shp, elt, "k_src"), _ptr(v_src, shp, elt, "v_src"), n_tok, _stream(stream))
    _check(st, "star_kv_write")


def star_attn_phase1(desc, k_cache, v_cache, q_ctx, o_ctx, stream=None):
    shp = (desc.batch, desc.ctx_len, desc.n_q_heads, desc.head_dim)
    elt = None if isinstance(q_ctx, int) else _elt(desc)
    st = load_library().star_attn_phase1(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        _ptr(q_ctx, shp, elt, "q_ctx"), _ptr(o_ctx, shp, elt, "o_ctx"), _stream(stream))
    _check(st, "star_attn_phase1")


def star_attn_phase2_plan(desc, kv_len: int, n_query: int) -> int:
    n = ctypes.c_int32(0)
    _check(load_library().star_attn_phase2_plan(ctypes.byref(desc), kv_len, n_query,
                                                ctypes.byref(n)), "star_attn_phase2_plan")
    return n.value


def star_attn_phase2_split_range(desc, kv_len: int, n_query: int, split: int) -> Tuple[int, int, int]:
    lo, hi, host = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    _check(load_library().star_attn_phase2_split_range(
        ctypes.byref(desc), kv_len, n_query, split, ctypes.byref(lo), ctypes.byref(hi),
        ctypes.byref(host)), "star_attn_phase2_split_range")
    return lo.value, hi.value, host.value


def star_attn_phase2_partial(desc, k_cache, v_cache, kv_len: int, q, n_query: int, o_part,
                             lse_part, stream=None):
    torch = None if isinstance(q, int) else _torch()
    n_split = star_attn_phase2_plan(desc, kv_len, n_query)
    shp_q = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    shp_o = (desc.batch, n_query, desc.n_q_heads, n_split, desc.head_dim)
    f32 = None if torch is None else torch.float32
    st = load_library().star_attn_phase2_partial(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        kv_len, _ptr(q, shp_q, None if torch is None else _elt(desc), "q"), n_query,
        _ptr(o_part, shp_o, f32, "o_part"), _ptr(lse_part, shp_o[:4], f32, "lse_part"),
        _stream(stream))
    _check(st, "star_attn_phase2_partial")


def star_attn_lse_merge(desc, n_query: int, n_split: int, o_part, lse_part, o, o_dtype: int,
                        lse_out=None, stream=None):
    torch = None if isinstance(o, int) else _torch()
    shp_o = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    f32 = None if torch is None else torch.float32
    od = None if torch is None else (torch.bfloat16 if o_dtype == STAR_BF16 else torch.float32)
    st = load_library().star_attn_lse_merge(
        ctypes.byref(desc), n_query, n_split,
        _ptr(o_part, shp_o[:3] + (n_split, desc.head_dim), f32, "o_part"),
        _ptr(lse_part, shp_o[:3] + (n_split,), f32, "lse_part"), _ptr(o, shp_o, od, "o"), o_dtype,
        _ptr(lse_out, shp_o[:3], f32, "lse_out"), _stream(stream))
    _check(st, "star_attn_lse_merge")


def star_attn_decode_step(desc, k_cache, v_cache, kv_len: int, q, k_new, v_new, n_query: int,
                          o_part, lse_part, o, o_dtype: int, lse_out=None, stream=None):
    torch = None if isinstance(q, int) else _torch()
    n_split = star_attn_phase2_plan(desc, kv_len, n_query)
    shp_q = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    shp_kv = (desc.batch, n_query, desc.n_kv_heads, desc.head_dim)
    shp_p = (desc.batch, n_query, desc.n_q_heads, n_split, desc.head_dim)
    f32 = None if torch is None else torch.float32
    elt = None if torch is None else _elt(desc)
    od = None if torch is None else (torch.bfloat16 if o_dtype == STAR_BF16 else torch.float32)
    st = load_library().star_attn_decode_step(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        kv_len, _ptr(q, shp_q, elt, "q"), _ptr(k_new, shp_kv, elt, "k_new"),
        _ptr(v_new, shp_kv, elt, "v_new"), n_query, _ptr(o_part, shp_p, f32, "o_part"),
        _ptr(lse_part, shp_p[:4], f32, "lse_part"), _ptr(o, shp_q, od, "o"), o_dtype, _ptr(lse_out, shp_q[:3], f32, "lse_out"), _stream(stream))
    _check(st, "star_attn_decode_step")


STAR_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/star_attn.h


def star_attn_decode_step_noalloc(desc, k_cache, v_cache, kv_len: int, q, k_new, v_new,
                                  n_query: int, o, o_dtype: int, lse_out=None, stream=None):
    """star_attn_decode_step with the split partials in the library's own
    per-GPU scratch array (the call allocates nothing)."""
    torch = None if isinstance(q, int) else _torch()
    shp_q = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    shp_kv = (desc.batch, n_query, desc.n_kv_heads, desc.head_dim)
    f32 = None if torch is None else torch.float32
    elt = None if torch is None else _elt(desc)
    od = None if torch is None else (torch.bfloat16 if o_dtype == STAR_BF16 else torch.float32)
    st = load_library().star_attn_decode_step_noalloc(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        kv_len, _ptr(q, shp_q, elt, "q"), _ptr(k_new, shp_kv, elt, "k_new"),
        _ptr(v_new, shp_kv, elt, "v_new"), n_query, _ptr(o, shp_q, od, "o"), o_dtype,
        _ptr(lse_out, shp_q[:3], f32, "lse_out"), _stream(stream))
    _check(st, "star_attn_decode_step_noalloc")


# ---------------------------------------------------------------- paged cache

def star_kv_page_bytes(desc: StarAttnDesc) -> int:
    return load_library().star_kv_page_bytes(ctypes.byref(desc))


def alloc_kv_pages(desc: StarAttnDesc, n_pages: int, device="cuda"):
    """A pool of n_pages K (or V) pages (torch.empty of n_pages * star_kv_page_bytes)."""
    torch = _torch()
    nbytes = star_kv_page_bytes(desc)
    if nbytes == 0 or n_pages < 1:
        raise StarAttnError(STAR_ERR_INVALID_ARG, "alloc_kv_pages")
    elt = _elt(desc)
    return torch.empty(n_pages * nbytes // torch.tensor([], dtype=elt).element_size(), dtype=elt,
                       device=device)


def _pages_ptr(desc, x, name):
    if isinstance(x, int) or x is None:
        return x
    nbytes = star_kv_page_bytes(desc)
    size = x.numel() * x.element_size()
    if nbytes == 0 or size < nbytes or size % nbytes:
        raise ValueError(f"{name}: {size} bytes is not a whole number of {nbytes}-byte pages")
    return _ptr(x, dtype=_elt(desc), name=name)


def _table(desc, block_table):
    """(pointer, max_pages) of a device int32 [batch][max_pages] table, or a
    (pointer, max_pages) pair passed through."""
    if isinstance(block_table, tuple):
        return block_table
    torch = _torch()
    if block_table.dim() != 2 or block_table.shape[0] != desc.batch:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)}, expected "
                         f"({desc.batch}, max_pages)")
    return _ptr(block_table, dtype=torch.int32, name="block_table"), int(block_table.shape[1])


def star_kv_write_paged(desc, k_pages, v_pages, block_table, pos0: int, k_src, v_src, n_tok: int,
                        stream=None):
    shp = (desc.batch, n_tok, desc.n_kv_heads, desc.head_dim)
    elt = None if isinstance(k_src, int) else _elt(desc)
    tp, mp = _table(desc, block_table)
    st = load_library().star_kv_write_paged(
        ctypes.byref(desc), _pages_ptr(desc, k_pages, "k_pages"), _pages_ptr(desc, v_pages, "v_pages"),
        tp, mp, pos0, _ptr(k_src, shp, elt, "k_src"), _ptr(v_src, shp, elt, "v_src"), n_tok,
        _stream(stream))
    _check(st, "star_kv_write_paged")


def star_attn_phase2_partial_paged(desc, k_pages, v_pages, block_table, kv_len: int, q,
                                   n_query: int, o_part, lse_part, stream=None):
    torch = None if isinstance(q, int) else _torch()
    n_split = star_attn_phase2_plan(desc, kv_len, n_query)
    shp_q = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    shp_o = (desc.batch, n_query, desc.n_q_heads, n_split, desc.head_dim)
    f32 = None if torch is None else torch.float32
    tp, mp = _table(desc, block_table)
    st = load_library().star_attn_phase2_partial_paged(
        ctypes.byref(desc), _pages_ptr(desc, k_pages, "k_pages"), _pages_ptr(desc, v_pages, "v_pages"),
        tp, mp, kv_len, _ptr(q, shp_q, None if torch is None else _elt(desc), "q"), n_query,
        _ptr(o_part, shp_o, f32, "o_part"), _ptr(lse_part, shp_o[:4], f32, "lse_part"),
        _stream(stream))
    _check(st, "star_attn_phase2_partial_paged")


def star_attn_decode_step_paged(desc, k_pages, v_pages, block_table, kv_len: int, q, k_new, v_new,
                                n_query: int, o_part, lse_part, o, o_dtype: int, lse_out=None,
                                stream=None):
    torch = None if isinstance(q, int) else _torch()
    n_split = star_attn_phase2_plan(desc, kv_len, n_query)
    shp_q = (desc.batch, n_query, desc.n_q_heads, desc.head_dim)
    shp_kv = (desc.batch, n_query, desc.n_kv_heads, desc.head_dim)
    shp_p = (desc.batch, n_query, desc.n_q_heads, n_split, desc.head_dim)
    f32 = None if torch is None else torch.float32
    elt = None if torch is None else _elt(desc)
    od = None if torch is None else (torch.bfloat16 if o_dtype == STAR_BF16 else torch.float32)
    tp, mp = _table(desc, block_table)
    st = load_library().star_attn_decode_step_paged(
        ctypes.byref(desc), _pages_ptr(desc, k_pages, "k_pages"), _pages_ptr(desc, v_pages, "v_pages"),
        tp, mp, kv_len, _ptr(q, shp_q, elt, "q"), _ptr(k_new, shp_kv, elt, "k_new"),
        _ptr(v_new, shp_kv, elt, "v_new"), n_query, _ptr(o_part, shp_p, f32, "o_part"),
        _ptr(lse_part, shp_p[:4], f32, "lse_part"), _ptr(o, shp_q, od, "o"), o_dtype,
        _ptr(lse_out, shp_q[:3], f32, "lse_out"), _stream(stream))
    _check(st, "star_attn_decode_step_paged")


# ---------------------------------------------------------------- rotary embedding

def make_rope(cos, sin, anchor_mode: int = STAR_ROPE_ORIGINAL) -> StarRope:
    """A ``star_rope`` over device fp32 tables ``[n_pos][head_dim/2]`` (torch
    tensors, which the caller keeps alive)."""
    torch = _torch()
    for name, t in (("cos", cos), ("sin", sin)):
        if t.dtype != torch.float32 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"rope {name}: a contiguous device float32 [n_pos, head_dim/2] tensor")
    if cos.shape != sin.shape:
        raise ValueError("rope: cos and sin differ in shape")
    return StarRope(cos.data_ptr(), sin.data_ptr(), int(cos.shape[0]), anchor_mode)


def _rope_arg(desc, rope):
    if rope is None:
        return None
    if not isinstance(rope, StarRope):
        raise TypeError("rope: a StarRope (make_rope)")
    return ctypes.byref(rope)


def star_kv_write_rope(desc, k_cache, v_cache, pos0: int, k_src, v_src, n_tok: int, rope,
                       stream=None):
    shp = (desc.batch, n_tok, desc.n_kv_heads, desc.head_dim)
    elt = None if isinstance(k_src, int) else _elt(desc)
    st = load_library().star_kv_write_rope(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        pos0, _ptr(k_src, shp, elt, "k_src"), _ptr(v_src, shp, elt, "v_src"), n_tok,
        _rope_arg(desc, rope), _stream(stream))
    _check(st, "star_kv_write_rope")


def star_attn_phase1_rope(desc, k_cache, v_cache, q_ctx, rope, o_ctx, stream=None):
    shp = (desc.batch, desc.ctx_len, desc.n_q_heads, desc.head_dim)
    elt = None if isinstance(q_ctx, int) else _elt(desc)
    st = load_library().star_attn_phase1_rope(
        ctypes.byref(desc), _cache_ptr(desc, k_cache, "k_cache"), _cache_ptr(desc, v_cache, "v_cache"),
        _ptr(q_ctx, shp, elt, "q_ctx"), _rope_arg(desc, rope), _ptr(o_ctx, shp, elt, "o_ctx"),
        _stream(stream))
    _check(st, "star_attn_phase1_rope")
