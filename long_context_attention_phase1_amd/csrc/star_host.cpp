// Host runtime of libstarattn: argument validation, the phase-2 split
// planner and the extern "C" entry points declared in include/star_attn.h.
// Pure C++ (no HIP calls), so every check here runs without a GPU; the
// kernel launches live in star_kernels.hip.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "star_internal.hpp"

namespace star {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

int validate_desc(const star_attn_desc* d, Dims* out) {
  if (!d) return STAR_ERR_INVALID_ARG;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->ctx_len < 1 ||
      d->block_len < 1 || d->anchor_len < 1 || d->tail_cap < 0)
    return STAR_ERR_INVALID_ARG;
  if (!(d->softmax_scale >= 0.0f) || isinf(d->softmax_scale)) return STAR_ERR_INVALID_ARG;
  if (d->dtype != STAR_BF16 && d->dtype != STAR_F32) return STAR_ERR_DTYPE;
  if (d->head_dim != 64 && d->head_dim != 128) return STAR_ERR_UNSUPPORTED;
  if (d->n_q_heads % d->n_kv_heads != 0) return STAR_ERR_SHAPE;
  if (d->anchor_len > d->block_len) return STAR_ERR_SHAPE;
  // keep every element index inside int64 and every grid inside 2^31 workgroups
  const int64_t rows = round_up(d->ctx_len + d->tail_cap, kTile);
  if (rows > ((int64_t)1 << 40) || (int64_t)d->batch * d->n_q_heads > (1 << 24))
    return STAR_ERR_SHAPE;
  // block indices are 32-bit
  if (cdiv(d->ctx_len, d->block_len) > INT32_MAX) return STAR_ERR_SHAPE;
  if (out) {
    Dims& o = *out;
    o.B = d->batch;
    o.Hq = d->n_q_heads;
    o.Hkv = d->n_kv_heads;
    o.G = d->n_q_heads / d->n_kv_heads;
    o.D = d->head_dim;
    o.L = d->ctx_len;
    o.blk = d->block_len;
    o.anc = d->anchor_len;
    o.tail_cap = d->tail_cap;
    o.rows = rows;
    o.n_blocks = (int32_t)cdiv(d->ctx_len, d->block_len);
    o.dtype = d->dtype;
    o.scale = d->softmax_scale == 0.0f ? (float)(1.0 / sqrt((double)d->head_dim))
                                       : d->softmax_scale;
    o.scale_log2 = (float)((double)o.scale * 1.4426950408889634);
    o.HW = (o.G % 4 == 0) ? 4 : (o.G % 2 == 0 ? 2 : 1);
    o.RW = kWaves / o.HW;
    o.HQ = o.G / o.HW;
  }
  return STAR_OK;
}

int validate_phase2(const Dims& d, int64_t kv_len, int64_t n_query) {
  if (n_query < 1) return STAR_ERR_INVALID_ARG;
  if (kv_len < d.L + 1 || kv_len > d.L + d.tail_cap) return STAR_ERR_SHAPE;
  if (n_query > kv_len - d.L) return STAR_ERR_SHAPE;
  return STAR_OK;
}

static int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Balanced decode plan (see Plan): equal ranges of whole 32-key slices, one
// per wave (four waves per workgroup, one workgroup per CU), at most one host
// boundary inside each. Returns false when the shape does not allow it.
static bool balanced_plan(const Dims& d, int64_t kv_len, Plan* p) {
  if (d.dtype != STAR_BF16) return false;
  const int64_t groups = (int64_t)d.B * d.Hkv;
  int64_t w = kDecodeWaves / groups;
  if (w < 1) w = 1;
  int64_t r = round_up(cdiv(kv_len, w), kSlice);
  if (r < kMinRange) r = kMinRange;
  w = cdiv(kv_len, r);
  int64_t n_split = 0;
  for (int64_t j = 0; j < w; ++j) {
    const int64_t a = j * r, b = a + r < kv_len ? a + r : kv_len;
    const int64_t bnd = inner_boundary(d.L, d.blk, d.n_blocks, a, b);
    if (bnd >= 0 && inner_boundary(d.L, d.blk, d.n_blocks, bnd, b) >= 0) return false;
    n_split += bnd >= 0 ? 2 : 1;
  }
  if (n_split > (1 << 20)) return false;
  p->balanced = 1;
  p->n_wg = (int32_t)w;
  p->wg_rows = r;
  p->bnd_period = r / gcd64(d.blk, r);
  p->n_split = (int32_t)n_split;
  return true;
}

Plan make_plan(const Dims& d, int64_t kv_len, int64_t n_query) {
  Plan p{};
  const int64_t cols = n_query * d.G;
  p.narrow = (d.dtype != STAR_BF16) || cols <= kNarrowCols;
  p.n_groups = p.narrow ? d.B * d.Hkv : d.B * d.Hkv * d.HQ;
  p.n_qtiles = p.narrow ? 1 : (int32_t)cdiv(n_query, (int64_t)kColsPerWave * d.RW);
  if (p.narrow && balanced_plan(d, kv_len, &p)) return p;
  // about one long-running workgroup per CU. Many query rows: every split
  // writes Tq x Hq x d fp32 partials that the merge reads back, so shorter
  // splits cost more partial traffic than they gain in balance (the 128K
  // query step: 0.33 ms at 257 splits per kv head, 0.21 ms at 33)
  const int64_t total = p.narrow ? kNarrowWorkgroups : kTargetWorkgroups;
  // fp32: one wave runs a split's 32-key slices one after another at the
  // matrix core's rate, so splits as short as a tile keep a short step's
  // chains parallel
  const int64_t min_len = d.dtype != STAR_BF16 ? kTile : (p.narrow ? 512 : 256);
  int64_t target = total / ((int64_t)p.n_groups * p.n_qtiles);
  if (target < 1) target = 1;
  // splits per context block: proportional to the block's share of the cache,
  // no split shorter than min_len rows
  int64_t per = (int64_t)llround((double)target * (double)d.blk / (double)kv_len);
  const int64_t max_per = d.blk / min_len;
  if (per > max_per) per = max_per;
  if (per <= 1) {
    p.per_block = 1;
    p.blk_len = d.blk;
  } else {
    p.blk_len = round_up(cdiv(d.blk, per), kTile);
    p.per_block = (int32_t)cdiv(d.blk, p.blk_len);
  }
  const int64_t tail = kv_len - d.L;
  const int64_t tl_target =
      p.per_block > 1 ? p.blk_len : (d.blk > min_len ? round_up(d.blk, kTile) : min_len);
  const int64_t tail_splits = cdiv(tail, tl_target);
  const int64_t n_split = (int64_t)d.n_blocks * p.per_block + tail_splits;
  if (n_split > INT32_MAX) {  // split ids are 32-bit: the caller refuses the shape
    p.n_split = 0;
    return p;
  }
  p.tail_splits = (int32_t)tail_splits;
  p.tail_len = p.tail_splits == 1 ? tail : round_up(cdiv(tail, p.tail_splits), kTile);
  p.n_split = (int32_t)n_split;
  return p;
}

// Every grid of a decode step (the append, the partials, the merge), checked
// before the first launch so that a call that fails writes nothing.
static int decode_step_fits(const Dims& d, const Plan& p, int64_t kv_len, int64_t n_query) {
  if (p.n_split < 1 || !partial_fits(d, p, n_query) || !merge_fits(d, n_query))
    return STAR_ERR_SHAPE;
  if (!fused_append(d, p) && !grid_fits(kv_write_grid(d, kv_len - n_query, n_query), 256))
    return STAR_ERR_SHAPE;
  return STAR_OK;
}

}  // namespace star

using namespace star;

extern "C" {

size_t star_kv_cache_bytes(const star_attn_desc* desc) {
  Dims d;
  if (validate_desc(desc, &d) != STAR_OK) return 0;
  const size_t elt = d.dtype == STAR_BF16 ? 2 : 4;
  return (size_t)d.B * d.Hkv * (size_t)d.rows * d.D * elt;
}

int star_kv_write(const star_attn_desc* desc, void* k_cache, void* v_cache, int64_t pos0,
                  const void* k_src, const void* v_src, int64_t n_tok, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !k_src || !v_src || n_tok < 1) return STAR_ERR_INVALID_ARG;
  if (pos0 < 0 || pos0 + n_tok > d.L + d.tail_cap) return STAR_ERR_SHAPE;
  if (!grid_fits(kv_write_grid(d, pos0, n_tok), 256)) return STAR_ERR_SHAPE;
  return launch_kv_write(d, k_cache, v_cache, pos0, k_src, v_src, n_tok, stream);
}

int star_attn_phase1(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                     const void* q_ctx, void* o_ctx, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !q_ctx || !o_ctx) return STAR_ERR_INVALID_ARG;
  if (!phase1_fits(d)) return STAR_ERR_SHAPE;
  return launch_phase1(d, k_cache, v_cache, q_ctx, o_ctx, stream);
}

int star_attn_phase2_plan(const star_attn_desc* desc, int64_t kv_len, int64_t n_query,
                          int32_t* n_split) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!n_split) return STAR_ERR_INVALID_ARG;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  if (p.n_split < 1) return STAR_ERR_SHAPE;
  *n_split = p.n_split;
  return STAR_OK;
}

int star_attn_phase2_split_range(const star_attn_desc* desc, int64_t kv_len, int64_t n_query,
                                 int32_t split, int64_t* lo, int64_t* hi, int32_t* host) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!lo || !hi || !host) return STAR_ERR_INVALID_ARG;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  if (p.n_split < 1 || split < 0 || split >= p.n_split) return STAR_ERR_SHAPE;
  split_range(d, p, kv_len, split, lo, hi, host);
  return STAR_OK;
}

int star_attn_phase2_partial(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                             int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                             float* lse_part, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !q || !o_part || !lse_part) return STAR_ERR_INVALID_ARG;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  if (p.n_split < 1 || !partial_fits(d, p, n_query)) return STAR_ERR_SHAPE;
  return launch_phase2_partial(d, p, k_cache, v_cache, kv_len, q, n_query, o_part, lse_part,
                               stream);
}

int star_attn_lse_merge(const star_attn_desc* desc, int64_t n_query, int32_t n_split,
                        const float* o_part, const float* lse_part, void* o, int32_t o_dtype,
                        float* lse_out, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!o_part || !lse_part || !o || n_query < 1 || n_split < 1) return STAR_ERR_INVALID_ARG;
  if (o_dtype != STAR_BF16 && o_dtype != STAR_F32) return STAR_ERR_DTYPE;
  if (n_query > d.tail_cap) return STAR_ERR_SHAPE;
  if (!merge_fits(d, n_query)) return STAR_ERR_SHAPE;
  return launch_lse_merge(d, n_query, n_split, o_part, lse_part, o, o_dtype, lse_out, stream);
}

int star_attn_decode_step(const star_attn_desc* desc, void* k_cache, void* v_cache,
                          int64_t kv_len, const void* q, const void* k_new, const void* v_new,
                          int64_t n_query, float* o_part, float* lse_part, void* o,
                          int32_t o_dtype, float* lse_out, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !q || !k_new || !v_new || !o_part || !lse_part || !o)
    return STAR_ERR_INVALID_ARG;
  if (o_dtype != STAR_BF16 && o_dtype != STAR_F32) return STAR_ERR_DTYPE;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  st = decode_step_fits(d, p, kv_len, n_query);
  if (st) return st;
  if (fused_append(d, p))
    return launch_decode_step(d, p, k_cache, v_cache, kv_len, q, k_new, v_new, n_query, o_part,
                              lse_part, o, o_dtype, lse_out, stream);
  // fp32, or several workgroups per split: the same three steps as separate
  // launches
  st = launch_kv_write(d, k_cache, v_cache, kv_len - n_query, k_new, v_new, n_query, stream);
  if (st) return st;
  st = launch_phase2_partial(d, p, k_cache, v_cache, kv_len, q, n_query, o_part, lse_part, stream);
  if (st) return st;
  return launch_lse_merge(d, n_query, p.n_split, o_part, lse_part, o, o_dtype, lse_out, stream);
}

int star_attn_decode_step_noalloc(const star_attn_desc* desc, void* k_cache, void* v_cache,
                                  int64_t kv_len, const void* q, const void* k_new,
                                  const void* v_new, int64_t n_query, void* o, int32_t o_dtype,
                                  float* lse_out, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !q || !k_new || !v_new || !o) return STAR_ERR_INVALID_ARG;
  if (o_dtype != STAR_BF16 && o_dtype != STAR_F32) return STAR_ERR_DTYPE;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  st = decode_step_fits(d, p, kv_len, n_query);
  if (st) return st;
  if (!noalloc_fits(d, p, n_query)) return STAR_ERR_SHAPE;
  void* base = nullptr;
  st = scratch_address(&base);
  if (st) return st;
  float* o_part = (float*)base;
  float* lse_part = (float*)((char*)base + noalloc_lse_offset(d, p, n_query));
  // the same launches as star_attn_decode_step, on the scratch partials
  if (fused_append(d, p))
    return launch_decode_step(d, p, k_cache, v_cache, kv_len, q, k_new, v_new, n_query, o_part,
                              lse_part, o, o_dtype, lse_out, stream);
  st = launch_kv_write(d, k_cache, v_cache, kv_len - n_query, k_new, v_new, n_query, stream);
  if (st) return st;
  st = launch_phase2_partial(d, p, k_cache, v_cache, kv_len, q, n_query, o_part, lse_part, stream);
  if (st) return st;
  return launch_lse_merge(d, n_query, p.n_split, o_part, lse_part, o, o_dtype, lse_out, stream);
}

// ---- paged cache: the same entry points, the cache read and written through a
// block table

size_t star_kv_page_bytes(const star_attn_desc* desc) {
  Dims d;
  if (validate_desc(desc, &d) != STAR_OK) return 0;
  const size_t elt = d.dtype == STAR_BF16 ? 2 : 4;
  return (size_t)d.Hkv * STAR_KV_TILE * d.D * elt;
}

// The page pools and a table that covers every row of the cache's capacity.
static int validate_pages(const Dims& d, const void* k_pages, const void* v_pages,
                          const int32_t* table, int32_t max_pages) {
  if (!k_pages || !v_pages || !table) return STAR_ERR_INVALID_ARG;
  if (max_pages < (d.L + d.tail_cap + STAR_KV_TILE - 1) / STAR_KV_TILE) return STAR_ERR_SHAPE;
  return STAR_OK;
}

int star_kv_write_paged(const star_attn_desc* desc, void* k_pages, void* v_pages,
                        const int32_t* block_table, int32_t max_pages, int64_t pos0,
                        const void* k_src, const void* v_src, int64_t n_tok, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_src || !v_src || n_tok < 1) return STAR_ERR_INVALID_ARG;
  st = validate_pages(d, k_pages, v_pages, block_table, max_pages);
  if (st) return st;
  if (pos0 < 0 || pos0 + n_tok > d.L + d.tail_cap) return STAR_ERR_SHAPE;
  if (!grid_fits(kv_write_grid(d, pos0, n_tok), 256)) return STAR_ERR_SHAPE;
  return launch_kv_write(d, k_pages, v_pages, pos0, k_src, v_src, n_tok, stream, block_table,
                         max_pages);
}

int star_attn_phase2_partial_paged(const star_attn_desc* desc, const void* k_pages,
                                   const void* v_pages, const int32_t* block_table,
                                   int32_t max_pages, int64_t kv_len, const void* q,
                                   int64_t n_query, float* o_part, float* lse_part, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!q || !o_part || !lse_part) return STAR_ERR_INVALID_ARG;
  st = validate_pages(d, k_pages, v_pages, block_table, max_pages);
  if (st) return st;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  if (p.n_split < 1 || !partial_fits(d, p, n_query)) return STAR_ERR_SHAPE;
  return launch_phase2_partial(d, p, k_pages, v_pages, kv_len, q, n_query, o_part, lse_part,
                               stream, block_table, max_pages);
}

int star_attn_decode_step_paged(const star_attn_desc* desc, void* k_pages, void* v_pages,
                                const int32_t* block_table, int32_t max_pages, int64_t kv_len,
                                const void* q, const void* k_new, const void* v_new,
                                int64_t n_query, float* o_part, float* lse_part, void* o,
                                int32_t o_dtype, float* lse_out, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!q || !k_new || !v_new || !o_part || !lse_part || !o) return STAR_ERR_INVALID_ARG;
  if (o_dtype != STAR_BF16 && o_dtype != STAR_F32) return STAR_ERR_DTYPE;
  st = validate_pages(d, k_pages, v_pages, block_table, max_pages);
  if (st) return st;
  st = validate_phase2(d, kv_len, n_query);
  if (st) return st;
  const Plan p = make_plan(d, kv_len, n_query);
  st = decode_step_fits(d, p, kv_len, n_query);
  if (st) return st;
  if (fused_append(d, p))
    return launch_decode_step(d, p, k_pages, v_pages, kv_len, q, k_new, v_new, n_query, o_part,
                              lse_part, o, o_dtype, lse_out, stream, block_table, max_pages);
  st = launch_kv_write(d, k_pages, v_pages, kv_len - n_query, k_new, v_new, n_query, stream,
                       block_table, max_pages);
  if (st) return st;
  st = launch_phase2_partial(d, p, k_pages, v_pages, kv_len, q, n_query, o_part, lse_part, stream,
                             block_table, max_pages);
  if (st) return st;
  return launch_lse_merge(d, n_query, p.n_split, o_part, lse_part, o, o_dtype, lse_out, stream);
}

// ---- rotary position embedding

static int validate_rope(const Dims& d, const star_rope* rope) {
  if (!rope || !rope->cos || !rope->sin) return STAR_ERR_INVALID_ARG;
  if (rope->anchor_mode != STAR_ROPE_ORIGINAL && rope->anchor_mode != STAR_ROPE_ADJACENT)
    return STAR_ERR_INVALID_ARG;
  if (rope->n_pos < d.L + d.tail_cap) return STAR_ERR_SHAPE;
  return STAR_OK;
}

int star_kv_write_rope(const star_attn_desc* desc, void* k_cache, void* v_cache, int64_t pos0,
                       const void* k_src, const void* v_src, int64_t n_tok,
                       const star_rope* rope, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !k_src || !v_src || n_tok < 1) return STAR_ERR_INVALID_ARG;
  st = validate_rope(d, rope);
  if (st) return st;
  if (pos0 < 0 || pos0 + n_tok > d.L + d.tail_cap) return STAR_ERR_SHAPE;
  if (!grid_fits(kv_write_grid(d, pos0, n_tok), 256)) return STAR_ERR_SHAPE;
  return launch_kv_write(d, k_cache, v_cache, pos0, k_src, v_src, n_tok, stream, nullptr, 0,
                         rope->cos, rope->sin);
}

int star_attn_phase1_rope(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                          const void* q_ctx, const star_rope* rope, void* o_ctx, void* stream) {
  Dims d;
  int st = validate_desc(desc, &d);
  if (st) return st;
  if (!k_cache || !v_cache || !q_ctx || !o_ctx) return STAR_ERR_INVALID_ARG;
  st = validate_rope(d, rope);
  if (st) return st;
  if (!phase1_fits(d)) return STAR_ERR_SHAPE;
  return launch_phase1(d, k_cache, v_cache, q_ctx, o_ctx, stream, rope->cos, rope->sin,
                       rope->anchor_mode);
}

const char* star_attn_strerror(int status) {
  switch (status) {
    case STAR_OK: return "success";
    case STAR_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or bad scale)";
    case STAR_ERR_SHAPE: return "inconsistent shape (heads, anchor/block, kv_len, n_query or cache range)";
    case STAR_ERR_DTYPE: return "unknown dtype";
    case STAR_ERR_UNSUPPORTED: return "unsupported head_dim (64 or 128)";
    case STAR_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int star_attn_abi_version(void) { return STAR_ATTN_ABI_VERSION; }

}  // extern "C"
