// Internal declarations shared by the host runtime (star_host.cpp) and the
// HIP kernels (star_kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/star_attn.h"

namespace star {

constexpr int kTile = STAR_KV_TILE;   // rows of a KV-cache tile
constexpr int kWaves = 4;             // waves per workgroup of the MFMA kernels
constexpr int kColsPerWave = 64;      // query columns (row, head pairs) per wave
constexpr int kNarrowCols = 32;       // columns of the single-tile decode kernel
constexpr int kTargetWorkgroups = 256;   // phase-2 planner target, many query rows (one per CU:
                                         // fewer, longer splits write fewer fp32 partials)
constexpr int kNarrowWorkgroups = 256;   // phase-2 planner target, decode (one per CU)
constexpr int kDecodeWaves = 4 * 256;    // balanced plan: ranges per launch (4 waves per CU)
constexpr int kSlice = 32;               // balanced plan: ranges are whole 32-key slices
constexpr int kMinRange = 128;           // balanced plan: shortest range

// Everything derived from a validated descriptor.
struct Dims {
  int32_t B, Hq, Hkv, G, D;
  int64_t L, blk, anc, tail_cap, rows;  // rows: cache rows per (seq, kv head)
  int32_t n_blocks;
  int32_t dtype;
  float scale;      // softmax scale
  float scale_log2; // scale * log2(e)
  // MFMA kernels: heads per workgroup (HW), 64-row sub-tiles per workgroup
  // (RW = 4 / HW), head sub-groups per kv head (HQ = G / HW).
  int32_t HW, RW, HQ;
};

// Phase-2 split plan: every split lies inside one host's share.
//
// Blockwise plan: each context block is cut into per_block splits of
// blk_len rows and the tail into tail_splits of tail_len rows; one workgroup
// per split.
//
// Balanced plan (decode kernel, bf16): the rows [0, kv_len) of every
// (sequence, kv head) are cut into n_wg equal ranges of wg_rows rows (whole
// 32-key slices), one wave each, four waves per workgroup, so that the whole
// grid is resident at once. A range holds at most one host boundary (a block
// start, or the context/tail edge), anywhere in it, on a slice edge or not;
// a range that holds one yields two splits, one on each side. Splits are
// numbered in row order.
struct Plan {
  int32_t narrow;         // 1: single-column-tile decode kernel, 0: wide kernel
  int32_t per_block;      // splits per context block
  int64_t blk_len;        // rows per block split
  int32_t tail_splits;    // splits of the tail [L, kv_len)
  int64_t tail_len;       // rows per tail split
  int32_t n_split;
  int32_t n_groups;       // workgroup groups (sequence, kv head[, head sub-group])
  int32_t n_qtiles;       // query-row tiles (wide kernel)
  int32_t balanced;       // 1: balanced plan
  int32_t n_wg;           // balanced: ranges (waves) per group
  int64_t wg_rows;        // balanced: rows per range
  int64_t bnd_period;     // balanced: block starts i*blk with i % bnd_period == 0 fall on a range edge
};

int validate_desc(const star_attn_desc* d, Dims* out);
int validate_phase2(const Dims& d, int64_t kv_len, int64_t n_query);
Plan make_plan(const Dims& d, int64_t kv_len, int64_t n_query);

#if defined(__HIPCC__)
#define STAR_HD __host__ __device__
#else
#define STAR_HD
#endif

// First host boundary strictly inside (lo, hi), or -1. Host boundaries are
// the block starts i*blk (1 <= i < n_blocks) and the tail start L.
STAR_HD static inline int64_t inner_boundary(int64_t L, int64_t blk, int32_t n_blocks, int64_t lo,
                                             int64_t hi) {
  const int64_t i = lo / blk + 1;
  if (i <= (int64_t)n_blocks - 1 && i * blk < hi) return i * blk;
  if (L > lo && L < hi) return L;
  return -1;
}

// Balanced plan: number of host boundaries below x that do not fall on a
// range edge (each adds one split before x).
STAR_HD static inline int64_t inner_boundaries_below(int64_t L, int64_t blk, int32_t n_blocks,
                                                     int64_t wg_rows, int64_t bnd_period,
                                                     int64_t x) {
  if (x <= 0) return 0;
  int64_t m = (x - 1) / blk;
  if (m > (int64_t)n_blocks - 1) m = (int64_t)n_blocks - 1;
  int64_t c = m - m / bnd_period;
  if (L < x && L % wg_rows != 0) ++c;
  return c;
}

// Split sigma of a plan -> rows [lo, hi) (lo == hi: empty) and host id
// (context block index, or n_blocks for the tail).
STAR_HD static inline void split_rows(int64_t L, int64_t blk, int32_t n_blocks, int32_t per_block,
                                      int64_t blk_len, int64_t tail_len, int64_t kv_len,
                                      int32_t sigma, int64_t* lo, int64_t* hi, int32_t* host) {
  const int64_t nb = (int64_t)n_blocks * per_block;
  if (sigma < nb) {
    const int64_t i = sigma / per_block, j = sigma % per_block;
    const int64_t bend = (i + 1) * blk < L ? (i + 1) * blk : L;
    int64_t a = i * blk + j * blk_len, b = a + blk_len;
    if (b > bend) b = bend;
    if (a > b) a = b;
    *lo = a; *hi = b; *host = (int32_t)i;
  } else {
    const int64_t t = sigma - nb;
    int64_t a = L + t * tail_len, b = a + tail_len;
    if (b > kv_len) b = kv_len;
    if (a > b) a = b;
    *lo = a; *hi = b; *host = n_blocks;
  }
}

static inline void split_range(const Dims& d, const Plan& p, int64_t kv_len, int32_t sigma,
                               int64_t* lo, int64_t* hi, int32_t* host) {
  if (!p.balanced) {
    split_rows(d.L, d.blk, d.n_blocks, p.per_block, p.blk_len, p.tail_len, kv_len, sigma, lo, hi,
               host);
    return;
  }
  // balanced plan: walk the ranges in row order, one or two splits each
  int64_t base = 0;
  for (int64_t j = 0; j < p.n_wg; ++j) {
    const int64_t a = j * p.wg_rows;
    const int64_t b = a + p.wg_rows < kv_len ? a + p.wg_rows : kv_len;
    const int64_t bnd = inner_boundary(d.L, d.blk, d.n_blocks, a, b);
    const int64_t n = bnd >= 0 ? 2 : 1;
    if (sigma < base + n) {
      const bool second = sigma == base + 1;
      *lo = second ? bnd : a;
      *hi = (bnd >= 0 && !second) ? bnd : b;
      *host = *lo < d.L ? (int32_t)(*lo / d.blk) : d.n_blocks;
      return;
    }
    base += n;
  }
  *lo = *hi = kv_len;
  *host = d.n_blocks;
}

// Kernel launchers (star_kernels.hip). Each returns STAR_OK or STAR_ERR_HIP.
// table / maxp: a paged cache (kc, vc the page pools; table [B][maxp] page
// ids), or null / 0 for the contiguous cache.
// rope_cos / rope_sin: rotary tables [n_pos][D/2] (K rotated at its cache
// row; phase 1's query at its position id, per rope_mode), or null.
int launch_kv_write(const Dims& d, void* kc, void* vc, int64_t pos0, const void* ks,
                    const void* vs, int64_t n_tok, void* stream, const int32_t* table = nullptr,
                    int32_t maxp = 0, const float* rope_cos = nullptr,
                    const float* rope_sin = nullptr);
int launch_phase1(const Dims& d, const void* kc, const void* vc, const void* q, void* o,
                  void* stream, const float* rope_cos = nullptr, const float* rope_sin = nullptr,
                  int rope_mode = 0);
int launch_phase2_partial(const Dims& d, const Plan& p, const void* kc, const void* vc,
                          int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                          float* lse_part, void* stream, const int32_t* table = nullptr,
                          int32_t maxp = 0);
int launch_decode_step(const Dims& d, const Plan& p, void* kc, void* vc, int64_t kv_len,
                       const void* q, const void* k_new, const void* v_new, int64_t n_query,
                       float* o_part, float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                       void* stream, const int32_t* table = nullptr, int32_t maxp = 0);
int launch_lse_merge(const Dims& d, int64_t n_query, int32_t n_split, const float* o_part,
                     const float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                     void* stream);

}  // namespace star
