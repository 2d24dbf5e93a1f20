/*
 * star_attn.h - C ABI of libstarattn, the MI355X (gfx950) hot path of
 * Star Attention's two-phase attention.
 *
 * Method (all pages are titled "Star Attention: Efficient LLM Inference over
 * Long Sequences"):
 *   Phase 1 - hotaipapers.com summary page, podcast transcript, Phase 1
 *     description: the context is cut into blocks, one per host; every block
 *     after the first is prefixed with the anchor block (a copy of the first
 *     block) and the hosts run local attention in parallel, with no
 *     communication. paperhub.cn rebuttal, reply to reviewer EMsM point 5 and
 *     to x5MA point 1: the attention is causal and the anchor is at most one
 *     block long (here: the first anchor_len rows of the context).
 *   Phase 2 - same podcast, Phase 2 description: the query reaches every
 *     host, each host attends over its own cached KV and replies with one
 *     vector and one scalar, and the query host aggregates the replies into
 *     global attention, appends to its KV cache and repeats per token.
 *     PMLR proceedings page, Abstract, and paperhub.cn reply to dnhh point 2:
 *     phase 2 attends densely to every cached token.
 *
 * Here the hosts are the context blocks of one GPU. The anchor's KV is never
 * copied and never cached twice: block i >= 1 reads rows [0, anchor_len) of
 * the one cache, which holds every context token exactly once.
 *
 * Conventions shared by every entry point
 *   - Status: STAR_OK (0) or a negative STAR_ERR_* code. Arguments are fully
 *     validated before anything is enqueued; on error nothing is launched and
 *     no output byte is written.
 *   - Memory: every buffer is caller-owned device memory (except desc and the
 *     small host outputs such as n_split). The library never allocates, frees
 *     or synchronises; its one piece of device memory is the static scratch
 *     array of star_attn_decode_step_noalloc. Buffers must be 16-byte aligned.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream). All work is
 *     enqueued asynchronously on it, in call order.
 *   - Thread safety: stateless and re-entrant; calls on different streams may
 *     run concurrently as long as they do not write the same buffers
 *     (star_attn_decode_step_noalloc writes its GPU's one scratch array).
 *   - Layouts are row-major C arrays; element types follow desc->dtype
 *     (bf16 = IEEE bfloat16 bit patterns, f32 = IEEE binary32) unless stated.
 */
#ifndef STAR_ATTN_H
#define STAR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STAR_ATTN_ABI_VERSION 1

/* Status codes. */
enum {
  STAR_OK = 0,
  STAR_ERR_INVALID_ARG = -1, /* null pointer, negative or zero size, bad scale */
  STAR_ERR_SHAPE = -2,       /* inconsistent sizes: Hq % Hkv, anchor > block, kv_len, n_query */
  STAR_ERR_DTYPE = -3,       /* unknown dtype code */
  STAR_ERR_UNSUPPORTED = -4, /* head_dim not in {64, 128} */
  STAR_ERR_HIP = -5          /* the HIP runtime rejected a launch */
};

/* Element types. */
enum { STAR_BF16 = 0, STAR_F32 = 1 };

/* Rows of one KV-cache tile; cache rows per (sequence, kv head) are rounded
 * up to a multiple of this. */
#define STAR_KV_TILE 64

/*
 * Problem description (sizes follow the pages' problem statement: context
 * length, block size, anchor size, query length; GQA head counts).
 *   batch        number of independent sequences, >= 1
 *   n_q_heads    query heads Hq, >= 1
 *   n_kv_heads   key/value heads Hkv, >= 1, Hq % Hkv == 0. Query head h reads
 *                kv head h / (Hq / Hkv) (consecutive query heads share one).
 *   head_dim     d, 64 or 128
 *   ctx_len      context tokens L, >= 1
 *   block_len    context block b, >= 1 (one host's share; the last block may
 *                be shorter when L % b != 0)
 *   anchor_len   a, 1 <= a <= b: rows [0, a) of the context form the anchor
 *   tail_cap     capacity of the query host's tail (query tokens plus
 *                generated tokens), >= 0; tail rows are [L, L + tail_cap)
 *   dtype        STAR_BF16 or STAR_F32: type of Q, K, V, O and the cache
 *   softmax_scale  multiplies q.k before the softmax; 0 selects 1/sqrt(d)
 */
typedef struct star_attn_desc {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t ctx_len;
  int64_t block_len;
  int64_t anchor_len;
  int64_t tail_cap;
  int32_t dtype;
  float softmax_scale;
} star_attn_desc;

/*
 * KV-cache layout (the block layout that every host reads; one buffer for
 * K and one for V, each star_kv_cache_bytes() bytes):
 *   R = round_up(ctx_len + tail_cap, STAR_KV_TILE) rows per (sequence, kv head)
 *   K element (s, g, r, e):  K[((s*Hkv + g)*R + r)*d + e]                 (row-major rows)
 *   V element (s, g, r, e):  V[((s*Hkv + g)*R + (r/64)*64)*d + e*64 + r%64] (each 64-row tile
 *                            stored dimension-major, i.e. transposed)
 * Rows [0, L) hold the context, block i being rows [i*b, min((i+1)*b, L));
 * rows [L, L + tail_cap) hold the tail. The anchor is rows [0, a).
 * Returns 0 when desc is invalid.
 */
size_t star_kv_cache_bytes(const star_attn_desc* desc);

/*
 * star_kv_write - copy n_tok token-major K/V rows into cache rows
 * [pos0, pos0 + n_tok) (the context once before phase 1; the query host's
 * appends in phase 2: podcast, Phase 2 description, cache update).
 *   k_src, v_src  [batch][n_tok][n_kv_heads][head_dim], desc->dtype
 *   k_cache, v_cache  the cache buffers described above
 * Requires 0 <= pos0 and pos0 + n_tok <= ctx_len + tail_cap, n_tok >= 1
 * (else STAR_ERR_SHAPE / STAR_ERR_INVALID_ARG). Rows outside the range are
 * left untouched. Bit-exact copy.
 */
int star_kv_write(const star_attn_desc* desc, void* k_cache, void* v_cache, int64_t pos0,
                  const void* k_src, const void* v_src, int64_t n_tok, void* stream);

/*
 * star_attn_phase1 - blockwise-local causal attention with the anchor block
 * (hotaipapers.com podcast, Phase 1 description; paperhub.cn reply to EMsM
 * point 5). For context row r of block i = r / b and query head h:
 *   keys(r) = [i*b, r]              if i == 0
 *   keys(r) = [0, a) U [i*b, r]     if i >= 1 (the anchor, then the block causally)
 *   o[r, h] = softmax(scale * q[r, h] . K[keys(r), g(h)]) . V[keys(r), g(h)]
 * One output per context token; anchor rows are not recomputed per block.
 *   q_ctx, o_ctx  [batch][ctx_len][n_q_heads][head_dim], desc->dtype
 *   k_cache, v_cache  cache with rows [0, ctx_len) already written
 * Accumulation is fp32; o is rounded once to desc->dtype.
 */
int star_attn_phase1(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                     const void* q_ctx, void* o_ctx, void* stream);

/*
 * star_attn_phase2_plan - number of key splits the partial kernel produces
 * for (kv_len, n_query). Deterministic in (desc, kv_len, n_query). Every
 * split lies inside one host's share: one context block, or the tail
 * [ctx_len, kv_len); splits may be empty. Same argument checks as
 * star_attn_phase2_partial.
 */
int star_attn_phase2_plan(const star_attn_desc* desc, int64_t kv_len, int64_t n_query,
                          int32_t* n_split);

/*
 * star_attn_phase2_split_range - rows [*lo, *hi) of split `split` under the
 * same plan, and *host = the context block it belongs to (ctx blocks
 * 0..n_blocks-1) or n_blocks for the tail. Host-only; no GPU work.
 */
int star_attn_phase2_split_range(const star_attn_desc* desc, int64_t kv_len, int64_t n_query,
                                 int32_t split, int64_t* lo, int64_t* hi, int32_t* host);

/*
 * star_attn_phase2_partial - per-host local attention of the query rows
 * (podcast, Phase 2 description: every host answers with one vector and one
 * scalar). Query j (0 <= j < n_query) sits at position p_j = kv_len - n_query + j,
 * its own K/V already written there, and sees cache rows [0, p_j]. For each
 * split [lo, hi) of the plan, query j and head h:
 *   o_part[s][j][h][split][:] = softmax over keys [lo, min(hi, p_j + 1)) (normalised), fp32
 *   lse_part[s][j][h][split]  = natural-log log-sum-exp of scale*q.k over the same keys
 * A split with no visible key writes o = 0 and lse = -inf.
 *   q         [batch][n_query][n_q_heads][head_dim], desc->dtype
 *   o_part    [batch][n_query][n_q_heads][n_split][head_dim] fp32
 *   lse_part  [batch][n_query][n_q_heads][n_split] fp32
 * Requires ctx_len + 1 <= kv_len <= ctx_len + tail_cap and
 * 1 <= n_query <= kv_len - ctx_len (query rows live in the tail).
 */
int star_attn_phase2_partial(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                             int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                             float* lse_part, void* stream);

/*
 * star_attn_lse_merge - the query host's aggregation (podcast, Phase 2
 * description) as an exact softmax renormalisation of the partials:
 *   m = max_s lse_s;  lse = m + ln sum_s exp(lse_s - m);  o = sum_s exp(lse_s - lse) o_s
 * Splits with lse = -inf get weight 0. fp32 arithmetic, one final rounding.
 *   o_part, lse_part  as written by star_attn_phase2_partial (n_split of its plan)
 *   o        [batch][n_query][n_q_heads][head_dim] of type o_dtype (STAR_BF16 / STAR_F32)
 *   lse_out  [batch][n_query][n_q_heads] fp32, or NULL
 */
int star_attn_lse_merge(const star_attn_desc* desc, int64_t n_query, int32_t n_split,
                        const float* o_part, const float* lse_part, void* o, int32_t o_dtype,
                        float* lse_out, void* stream);

/*
 * star_attn_decode_step - one step of the query host's autoregressive loop
 * (podcast, Phase 2 description: append the new token's KV to the cache,
 * gather every host's vector and scalar, aggregate):
 *   1. writes k_new / v_new ([batch][n_query][n_kv_heads][head_dim], desc->dtype)
 *      into cache rows [kv_len - n_query, kv_len);
 *   2. computes the split partials exactly as star_attn_phase2_partial
 *      (o_part, lse_part laid out as there, n_split from star_attn_phase2_plan);
 *   3. merges them exactly as star_attn_lse_merge into o / lse_out.
 * When n_query * (n_q_heads / n_kv_heads) <= 32 and dtype is bf16, steps 1
 * and 2 are one kernel launch (the split that owns the new rows writes them
 * before reading them) and step 3 a second; otherwise three launches (a
 * query step of many tokens is one call too).
 * Argument checks as the three separate calls.
 */
int star_attn_decode_step(const star_attn_desc* desc, void* k_cache, void* v_cache,
                          int64_t kv_len, const void* q, const void* k_new, const void* v_new,
                          int64_t n_query, float* o_part, float* lse_part, void* o,
                          int32_t o_dtype, float* lse_out, void* stream);

/*
 * Paged KV cache (paperhub.cn rebuttal, reply to reviewer dKGV point 3,
 * serving frameworks: a paged memory manager can hold each host's local KV
 * cache). The same phase-2 operations with the cache kept in pages of
 * STAR_KV_TILE rows, found through a block table; phase 1 reads the
 * contiguous cache described above.
 *   k_pages, v_pages  pools of pages; page p holds, for every kv head g,
 *                the tile in the contiguous layout's form:
 *                K element (p, g, r, e): K[((p*Hkv + g)*64 + r)*d + e]
 *                V element (p, g, r, e): V[((p*Hkv + g)*64)*d + e*64 + r]
 *                (star_kv_page_bytes() bytes per page and per pool)
 *   block_table  device int32 [batch][max_pages]: entry [s][t] is the page
 *                holding rows [64t, 64t + 64) of sequence s.
 *                max_pages >= ceil((ctx_len + tail_cap) / 64) (else
 *                STAR_ERR_SHAPE). Every entry for rows a call reads or writes
 *                must be a valid page of the pools; the library cannot check
 *                device memory, and an invalid id is undefined behaviour.
 *                Sequences may share pages they only read (a common prefix);
 *                rows that are written must not share a page with rows
 *                another sequence or call reads at the same time.
 * Results are bit-identical to the contiguous-cache calls on the same
 * values: only the addresses differ.
 */
size_t star_kv_page_bytes(const star_attn_desc* desc);

/* star_kv_write through the block table (same arguments, checks and copy). */
int star_kv_write_paged(const star_attn_desc* desc, void* k_pages, void* v_pages,
                        const int32_t* block_table, int32_t max_pages, int64_t pos0,
                        const void* k_src, const void* v_src, int64_t n_tok, void* stream);

/* star_attn_phase2_partial on the paged cache (same plan and outputs). */
int star_attn_phase2_partial_paged(const star_attn_desc* desc, const void* k_pages,
                                   const void* v_pages, const int32_t* block_table,
                                   int32_t max_pages, int64_t kv_len, const void* q,
                                   int64_t n_query, float* o_part, float* lse_part,
                                   void* stream);

/* star_attn_decode_step on the paged cache (same steps, launches and outputs). */
int star_attn_decode_step_paged(const star_attn_desc* desc, void* k_pages, void* v_pages,
                                const int32_t* block_table, int32_t max_pages, int64_t kv_len,
                                const void* q, const void* k_new, const void* v_new,
                                int64_t n_query, float* o_part, float* lse_part, void* o,
                                int32_t o_dtype, float* lse_out, void* stream);

/*
 * Rotary position embedding fused into phase 1, with the anchor's position
 * ids (paperhub.cn rebuttal, reply to reviewer x5MA point 1: with the first
 * block as the anchor, the position ids given to the anchor tokens in
 * phase 1 change the result little). The pages name no scheme; this is the
 * rotary embedding of the Llama models they evaluate, half-split pairing:
 * element e < d/2 of a head vector turns together with element e + d/2,
 *   y_e = x_e c - x_{e+d/2} s,   y_{e+d/2} = x_{e+d/2} c + x_e s,
 * with (c, s) = (cos[pos][e], sin[pos][e]) from the caller's tables (any
 * frequency schedule). Arithmetic is fp32, each product and sum rounded on
 * its own; bf16 results are rounded once to nearest even (the rotated keys
 * a bf16 model caches).
 *   cos, sin     device fp32 tables [n_pos][head_dim / 2], 16-byte aligned
 *   n_pos        rows of the tables; >= ctx_len + tail_cap (else
 *                STAR_ERR_SHAPE)
 *   anchor_mode  position ids of anchor row j (j < anchor_len) as block
 *                i >= 1 sees it:
 *                STAR_ROPE_ORIGINAL  j, its place in the context;
 *                STAR_ROPE_ADJACENT  i*block_len - anchor_len + j, directly
 *                                    before the block.
 *                Every other key and every query keeps its context row.
 */
enum { STAR_ROPE_ORIGINAL = 0, STAR_ROPE_ADJACENT = 1 };

typedef struct star_rope {
  const float* cos;
  const float* sin;
  int64_t n_pos;
  int32_t anchor_mode;
} star_rope;

/* star_kv_write with each K row rotated at its cache row pos0 + t (V is
 * copied unchanged). The contiguous cache; same arguments and checks. */
int star_kv_write_rope(const star_attn_desc* desc, void* k_cache, void* v_cache, int64_t pos0,
                       const void* k_src, const void* v_src, int64_t n_tok,
                       const star_rope* rope, void* stream);

/* star_attn_phase1 with q_ctx not yet rotated: each query is rotated at its
 * context row, and for the anchor pass of block i >= 1 at the row less
 * (i*block_len - anchor_len) under STAR_ROPE_ADJACENT (rotations compose, so
 * this equals keeping the query and giving the anchor rows the adjacent
 * ids). The cache holds K rotated at its rows (star_kv_write_rope). */
int star_attn_phase1_rope(const star_attn_desc* desc, const void* k_cache, const void* v_cache,
                          const void* q_ctx, const star_rope* rope, void* o_ctx, void* stream);

/*
 * star_attn_decode_step_noalloc - star_attn_decode_step for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The same arguments less o_part and
 * lse_part: the split partials live in a scratch array that the library
 * holds in device memory, STAR_NOALLOC_SCRATCH_BYTES on each GPU it runs on,
 * from the first call on that GPU until the process ends. The call allocates
 * nothing, computes exactly what star_attn_decode_step computes (same kernels,
 * same plan, bit-identical o and lse_out), and returns STAR_ERR_SHAPE when the
 * partials do not fit the scratch (B * n_query * n_q_heads * n_split splits of
 * head_dim + 1 floats each, the o part rounded up to 256 bytes). Every call on
 * one GPU shares that GPU's scratch, which keeps the last call's partials:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * ordered by the caller. Returns STAR_ERR_HIP if the scratch's device address
 * cannot be looked up on the current device.
 */
#define STAR_NOALLOC_SCRATCH_BYTES (16u << 20)
int star_attn_decode_step_noalloc(const star_attn_desc* desc, void* k_cache, void* v_cache,
                                  int64_t kv_len, const void* q, const void* k_new,
                                  const void* v_new, int64_t n_query, void* o, int32_t o_dtype,
                                  float* lse_out, void* stream);

/* Human-readable text for a status code (static storage). */
const char* star_attn_strerror(int status);

/* STAR_ATTN_ABI_VERSION of the loaded library. */
int star_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STAR_ATTN_H */
