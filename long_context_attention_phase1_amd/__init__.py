"""Star Attention two-phase attention hot path for MI355X (gfx950).

The compute lives in ``libstarattn.so`` (hand-written HIP kernels behind the
C ABI of ``include/star_attn.h``); ``binding`` exposes the same entry points
to Python over PyTorch device tensors. ``synthetic`` draws seeded inputs.
"""
from .binding import (STAR_BF16, STAR_F32, STAR_OK, StarAttnDesc, StarAttnError,  # noqa: F401
                      alloc_kv_cache, alloc_kv_pages, load_library, make_desc,
                      star_attn_abi_version, star_attn_decode_step, star_attn_decode_step_noalloc,
                      star_attn_decode_step_paged,
                      star_attn_lse_merge, star_attn_phase1, star_attn_phase2_partial,
                      star_attn_phase2_partial_paged, star_attn_phase2_plan,
                      star_attn_phase2_split_range, star_attn_strerror, star_kv_cache_bytes,
                      star_kv_page_bytes, star_kv_write, star_kv_write_paged,
                      STAR_ROPE_ADJACENT, STAR_ROPE_ORIGINAL, StarRope, make_rope,
                      star_attn_phase1_rope, star_kv_write_rope)
