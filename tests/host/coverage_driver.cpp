// Host replay of every kernel launch's workgroup -> work mapping.
//
// For each shape read from stdin (one per line:
//   name B Hq Hkv d L block anchor n_query n_decode dtype(0 bf16, 1 f32)),
// the driver computes the launch geometry and walks every workgroup (and
// every wave and lane of it) through the same STAR_HD maps the kernels call
// on blockIdx (star_internal.hpp), then checks:
//   * phase 1: every (sequence, context row, query head) output is written by
//     exactly one lane; every work item (group, block, row tile) is taken by
//     exactly one workgroup; the key tiles of a workgroup cover exactly the
//     anchor [0, a) (blocks i >= 1) and the block's rows up to the last query
//     row, interior tiles only where every query of the workgroup sees all 64
//     keys; every tile lies inside the cache buffer and inside the written
//     context rows;
//   * the phase-2 query step and decode steps at several lengths: every
//     (sequence, query, head, split) partial is written exactly once; each
//     split's rows are those the host-side plan gives it; every loaded row
//     lies inside the cache and below kv_len; the appended rows of a fused
//     decode step are written once;
//   * the fp32 kernel: every output or partial is written by one column of
//     one wave, each column's keys are the method's key set, and every
//     loaded slice lies inside the written cache rows.
// No GPU; run by tests/test_work_coverage.py.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "star_internal.hpp"

namespace star {
// the entry points of star_host.cpp link against these; the replay calls none
int launch_kv_write(const Dims&, void*, void*, int64_t, const void*, const void*, int64_t, void*,
                    const int32_t*, int32_t, const float*, const float*) { return STAR_ERR_HIP; }
int launch_phase1(const Dims&, const void*, const void*, const void*, void*, void*, const float*,
                  const float*, int) { return STAR_ERR_HIP; }
int launch_phase2_partial(const Dims&, const Plan&, const void*, const void*, int64_t,
                          const void*, int64_t, float*, float*, void*, const int32_t*, int32_t) {
  return STAR_ERR_HIP;
}
int launch_decode_step(const Dims&, const Plan&, void*, void*, int64_t, const void*, const void*,
                       const void*, int64_t, float*, float*, void*, int32_t, float*, void*,
                       const int32_t*, int32_t) { return STAR_ERR_HIP; }
int launch_lse_merge(const Dims&, int64_t, int32_t, const float*, const float*, void*, int32_t,
                     float*, void*) { return STAR_ERR_HIP; }
int scratch_address(void**) { return STAR_ERR_HIP; }
}  // namespace star

using namespace star;

static int g_fail = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      if (g_fail < 20) std::fprintf(stderr, "%s: check failed line %d: %s\n", \
                                    g_name.c_str(), __LINE__, #c);            \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

static std::string g_name;

// A bit per item; counts how many items were set twice.
struct Bits {
  std::vector<uint64_t> w;
  int64_t n = 0, dup = 0, set = 0;
  explicit Bits(int64_t n_) : w((size_t)((n_ + 63) / 64), 0), n(n_) {}
  void mark(int64_t i) {
    if (i < 0 || i >= n) {
      ++dup;  // out of range counts as a failure too
      return;
    }
    uint64_t& x = w[(size_t)(i >> 6)];
    const uint64_t b = 1ull << (i & 63);
    if (x & b) ++dup;
    else ++set;
    x |= b;
  }
};

// the 64-row tile t of (sequence s, kv head g) inside the cache buffer
static void check_tile(const Dims& d, int s, int g, int64_t t) {
  CHECK(t >= 0 && 64 * (t + 1) <= d.rows);
  const int64_t e0 = (((int64_t)s * d.Hkv + g) * d.rows + 64 * t) * d.D;
  const int64_t total = (int64_t)d.B * d.Hkv * d.rows * d.D;
  CHECK(e0 >= 0 && e0 + 64 * d.D <= total);
}

// Keys one workgroup reads with its tile runs: interior tiles whole, edge
// tiles only their keys inside the given range. Checks the runs cover exactly
// [0, hiA) and [loB, hiB), each key once, interior keys visible to every
// query (at or before min_pos), and every loaded key below `written`.
static void check_runs(const Dims& d, int s, int g, const TileRuns& tr, int64_t hiA, int64_t loB,
                       int64_t hiB, int64_t min_pos, int64_t written) {
  // anchor
  CHECK(64 * tr.nAi <= hiA);
  CHECK(tr.a_edge ? (hiA > 64 * tr.nAi && hiA < 64 * (tr.nAi + 1)) : hiA == 64 * tr.nAi);
  for (int64_t t = 0; t < tr.nAi + (tr.a_edge ? 1 : 0); ++t) check_tile(d, s, g, t);
  CHECK(hiA <= written);
  if (hiB <= loB) {
    CHECK(tr.bf == 0 && tr.bl == 0 && tr.i0 == 0 && tr.i1 == 0);
    return;
  }
  // block: [bf, bl) tiles, interior [i0, i1) inside, edges around it
  CHECK(tr.bf == loB / 64 && tr.bl == (hiB + 63) / 64);
  CHECK(tr.bf <= tr.i0 && tr.i0 <= tr.i1 && tr.i1 <= tr.bl);
  if (tr.i1 > tr.i0) {
    CHECK(64 * tr.i0 >= loB);
    CHECK(64 * tr.i1 <= hiB);
    CHECK(64 * tr.i1 - 1 <= min_pos);
  }
  for (int64_t t = tr.bf; t < tr.bl; ++t) check_tile(d, s, g, t);
  // anchor and block keys disjoint
  CHECK(hiA <= loB);
  CHECK(hiB <= written);
}

// ---- phase 1 -------------------------------------------------------------

static void replay_phase1(const Dims& d) {
  const WideGeom gm = phase1_geom(d);
  const int QT = 8 / kWideWaves;
  Bits outs((int64_t)d.B * d.L * d.Hq);
  Bits items((int64_t)gm.NG * gm.n_blocks * gm.NRT);
  int64_t idle = 0;
  for (int64_t bid = 0; bid < gm.grid; ++bid) {
    int32_t gidx;
    int64_t work;
    wide_map(bid, true, gm.NG, gm.HQ, gm.NRT, gm.n_split, gm.n_blocks, &gidx, &work);
    CHECK(gidx >= 0 && gidx < gm.NG && work >= 0 && work < (int64_t)gm.n_blocks * gm.NRT);
    const int hq = gidx % gm.HQ, t2 = gidx / gm.HQ;
    const int kvh = t2 % d.Hkv, s = t2 / d.Hkv;
    CHECK(s < d.B);
    int64_t i, rt;
    phase1_item(work, gm.n_blocks, gm.NRT, &i, &rt);
    CHECK(i >= 0 && i < d.n_blocks && rt >= 0 && rt < gm.NRT);
    items.mark(((int64_t)gidx * gm.n_blocks + i) * gm.NRT + rt);
    const int64_t row0 = i * d.blk + rt * gm.BM;
    const int64_t row_end = (i + 1) * d.blk < d.L ? (i + 1) * d.blk : d.L;
    if (row0 >= row_end) {
      ++idle;  // the kernel returns at once (ragged last block)
      continue;
    }
    const int64_t hiA = i > 0 ? d.anc : 0;
    const int64_t loB = i * d.blk;
    const int64_t hiB = row0 + gm.BM < row_end ? row0 + gm.BM : row_end;
    const TileRuns tr = tile_runs(hiA, loB, hiB, row0);
    check_runs(d, s, kvh, tr, hiA, loB, hiB, row0, d.L);
    for (int w = 0; w < kWideWaves; ++w) {
      int hw;
      int64_t off;
      wide_wave(w, QT, d.HW, false, &hw, &off);
      const int head = kvh * d.G + hq * d.HW + hw;
      CHECK(head >= 0 && head < d.Hq);
      for (int qt = 0; qt < QT; ++qt)
        for (int l = 0; l < 32; ++l) {
          const int64_t r = row0 + off + 32 * qt + l;
          if (r >= row_end) continue;
          CHECK(r >= i * d.blk && r < hiB);
          outs.mark(((int64_t)s * d.L + r) * d.Hq + head);
        }
    }
  }
  CHECK(items.dup == 0 && items.set == items.n);
  CHECK(outs.dup == 0 && outs.set == outs.n);
  std::printf("  phase 1: %lld workgroups (%lld idle), %lld outputs once each\n",
              (long long)gm.grid, (long long)idle, (long long)outs.set);
}

// ---- phase 2 -------------------------------------------------------------

// the plan's split sigma, from the host-side walk
static void plan_split(const Dims& d, const Plan& p, int64_t kv_len, int32_t sigma, int64_t* lo,
                       int64_t* hi) {
  int32_t host;
  split_range(d, p, kv_len, sigma, lo, hi, &host);
}

static void replay_wide2(const Dims& d, const Plan& p, int64_t kv_len, int64_t n_query) {
  const WideGeom gm = wide2_geom(d, p);
  const int QT = 8 / kWideWaves;
  Bits parts((int64_t)d.B * n_query * d.Hq * p.n_split);
  CHECK(!fused_append(d, p));  // the wide kernel never appends
  const int64_t pos_off = kv_len - n_query;
  const bool short_tile = wide2_short(gm, n_query);  // the waves past row 32 hold no live row
  CHECK(!short_tile || (gm.NRT == 1 && 2 * n_query <= gm.BM));
  for (int64_t bid = 0; bid < gm.grid; ++bid) {
    int32_t gidx;
    int64_t work;
    wide_map(bid, false, gm.NG, gm.HQ, gm.NRT, gm.n_split, gm.n_blocks, &gidx, &work);
    CHECK(gidx >= 0 && gidx < gm.NG);
    const int hq = gidx % gm.HQ, t2 = gidx / gm.HQ;
    const int kvh = t2 % d.Hkv, s = t2 / d.Hkv;
    CHECK(s < d.B);
    const int64_t qrt = work % gm.NRT;
    const int32_t sigma = (int32_t)(work / gm.NRT);
    CHECK(sigma >= 0 && sigma < p.n_split);
    const int64_t row0 = qrt * gm.BM;
    if (row0 >= n_query) continue;
    int64_t loB, hiB;
    int32_t host;
    split_rows(d.L, d.blk, d.n_blocks, p.per_block, p.blk_len, p.tail_len, kv_len, sigma, &loB,
               &hiB, &host);
    int64_t plo, phi;
    plan_split(d, p, kv_len, sigma, &plo, &phi);
    CHECK(loB == plo && hiB == phi);
    const TileRuns tr = tile_runs(0, loB, hiB, row0 + pos_off);
    check_runs(d, s, kvh, tr, 0, loB, hiB, row0 + pos_off, kv_len);
    for (int w = 0; w < kWideWaves; ++w) {
      int hw;
      int64_t off;
      wide_wave(w, QT, d.HW, short_tile, &hw, &off);
      const int head = kvh * d.G + hq * d.HW + hw;
      CHECK(head >= 0 && head < d.Hq);
      for (int qt = 0; qt < QT; ++qt)
        for (int l = 0; l < 32; ++l) {
          const int64_t r = row0 + off + 32 * qt + l;
          if (r >= n_query) continue;
          parts.mark((((int64_t)s * n_query + r) * d.Hq + head) * p.n_split + sigma);
        }
    }
  }
  CHECK(parts.dup == 0 && parts.set == parts.n);
}

// decode kernel (balanced plan), fused with the append
static void replay_decode(const Dims& d, const Plan& p, int64_t kv_len, int64_t n_query) {
  int32_t wpg;
  const int64_t grid = decode_grid(d, p, &wpg);
  const int32_t NG = d.B * d.Hkv;
  const int64_t pos0 = kv_len - n_query;
  Bits splits((int64_t)NG * p.n_split);
  Bits appended((int64_t)NG * n_query);
  for (int64_t bid = 0; bid < grid; ++bid)
    for (int w = 0; w < 4; ++w) {
      int32_t gidx;
      int64_t r;
      decode_map(bid, w, NG, wpg, &gidx, &r);
      CHECK(gidx >= 0 && gidx < NG && r >= 0);
      if (r >= p.n_wg) continue;
      const int kvh = gidx % d.Hkv, s = gidx / d.Hkv;
      const DecodeRange rg =
          decode_range(r, p.wg_rows, kv_len, d.L, d.blk, d.n_blocks, p.bnd_period, pos0);
      CHECK(rg.lo < rg.hi && rg.hi <= kv_len);
      CHECK(rg.n_sl == (rg.hi - rg.lo + 31) / 32);
      CHECK(rg.n_in >= 0 && rg.n_in <= rg.n_sl && rg.lo + 32 * rg.n_in <= pos0 + 1);
      // its split(s) match the plan's rows
      int64_t plo, phi;
      if (rg.bnd >= 0) {
        CHECK(rg.bnd > rg.lo && rg.bnd < rg.hi);
        plan_split(d, p, kv_len, rg.sigma, &plo, &phi);
        CHECK(plo == rg.lo && phi == rg.bnd);
        plan_split(d, p, kv_len, rg.sigma + 1, &plo, &phi);
        CHECK(plo == rg.bnd && phi == rg.hi);
        splits.mark((int64_t)gidx * p.n_split + rg.sigma + 1);
      } else {
        plan_split(d, p, kv_len, rg.sigma, &plo, &phi);
        CHECK(plo == rg.lo && phi == rg.hi);
      }
      splits.mark((int64_t)gidx * p.n_split + rg.sigma);
      // slices: K rows [lo + 32 i, + 32) and the V^T tile holding them
      for (int i = 0; i < rg.n_sl; ++i) {
        const int64_t row = rg.lo + 32 * (int64_t)i;
        CHECK(row < kv_len);
        check_tile(d, s, kvh, row / 64);
      }
      // the append: this range's share of the new rows
      const int64_t a0 = pos0 > rg.lo ? pos0 : rg.lo, a1 = kv_len < rg.hi ? kv_len : rg.hi;
      for (int64_t row = a0; row < a1; ++row) appended.mark((int64_t)gidx * n_query + (row - pos0));
    }
  CHECK(splits.dup == 0 && splits.set == splits.n);
  CHECK(appended.dup == 0 && appended.set == appended.n);
}

// narrow kernel (blockwise plan)
static void replay_narrow(const Dims& d, const Plan& p, int64_t kv_len, int64_t n_query) {
  const int32_t NG = d.B * d.Hkv;
  const int64_t pos0 = kv_len - n_query;
  Bits splits((int64_t)NG * p.n_split);
  Bits appended((int64_t)NG * n_query);
  for (int64_t bid = 0; bid < (int64_t)NG * p.n_split; ++bid) {
    int32_t gidx, sigma;
    narrow_map(bid, NG, p.n_split, &gidx, &sigma);
    CHECK(gidx >= 0 && gidx < NG && sigma >= 0 && sigma < p.n_split);
    splits.mark((int64_t)gidx * p.n_split + sigma);
    const int kvh = gidx % d.Hkv, s = gidx / d.Hkv;
    int64_t lo, hi;
    int32_t host;
    split_rows(d.L, d.blk, d.n_blocks, p.per_block, p.blk_len, p.tail_len, kv_len, sigma, &lo, &hi,
               &host);
    const TileRuns tr = tile_runs(0, lo, hi, pos0);
    check_runs(d, s, kvh, tr, 0, lo, hi, pos0, kv_len);
    const int64_t a0 = pos0 > lo ? pos0 : lo, a1 = kv_len < hi ? kv_len : hi;
    for (int64_t row = a0; row < a1; ++row) appended.mark((int64_t)gidx * n_query + (row - pos0));
  }
  CHECK(splits.dup == 0 && splits.set == splits.n);
  CHECK(appended.dup == 0 && appended.set == appended.n);
}

// fp32 MFMA kernel: one wave per 32 columns (phase 1: rows of a head;
// phase 2: (query, head) pairs of a kv head, one split)
static void replay_f32m(const Dims& d, bool phase1, const Plan* p, int64_t kv_len,
                        int64_t n_query) {
  const int64_t q_tokens = phase1 ? d.L : n_query;
  const int64_t ncg = phase1 ? 0 : f32m_ncg(d, n_query);
  const int64_t grid = phase1 ? f32m_phase1_grid(d) : f32m_phase2_grid(d, *p, n_query);
  const int64_t n_out = phase1 ? (int64_t)d.B * d.L * d.Hq
                               : (int64_t)d.B * n_query * d.Hq * p->n_split;
  const int64_t written = phase1 ? d.L : kv_len;
  Bits outs(n_out);
  for (int64_t wid = 0; wid < grid; ++wid) {
    int64_t s, rg = 0, cg = 0, lo = 0, hi = 0;
    int32_t h = 0, kvh = 0, sigma = 0;
    if (phase1) {
      f32m_phase1_map(wid, d.L, d.Hq, &s, &h, &rg);
      kvh = h / d.G;
    } else {
      f32m_phase2_map(wid, p->n_split, ncg, d.Hkv, &s, &kvh, &cg, &sigma);
      int32_t host;
      split_rows(d.L, d.blk, d.n_blocks, p->per_block, p->blk_len, p->tail_len, kv_len, sigma, &lo,
                 &hi, &host);
      int64_t plo, phi;
      plan_split(d, *p, kv_len, sigma, &plo, &phi);
      CHECK(lo == plo && hi == phi);
    }
    CHECK(s >= 0 && s < d.B && kvh >= 0 && kvh < d.Hkv && sigma >= 0);
    const int64_t gsel = phase1 ? rg : cg;
    const int32_t hsel = phase1 ? h : kvh;
    int64_t kA, kB0, kB1;
    f32m_wave_keys(phase1, gsel, hsel, d.L, d.blk, d.anc, q_tokens, d.G, kv_len, lo, hi, &kA, &kB0,
                   &kB1);
    // the loaded rows: the wanted keys of the processed slices, all written
    const int64_t k_end = kA > kB1 ? kA : kB1;
    CHECK(kA <= written && kB1 <= written);
    // the closed-form slice list is exactly the slices f32m_slice accepts, in
    // order, and the round-robin deal gives each to one wave
    const F32mSlices sl = f32m_slices(kA, kB0, kB1);
    const int NW = f32m_waves(d.D);
    int64_t n_seen = 0;
    for (int64_t k0 = 0; k0 < k_end; k0 += 32) {
      if (!f32m_slice(k0, kA, kB0, kB1)) continue;
      CHECK(n_seen < sl.n && f32m_slice_at(sl, n_seen) == k0);
      check_tile(d, (int)s, kvh, k0 / 64);
      ++n_seen;
    }
    CHECK(n_seen == sl.n);
    int64_t dealt = 0;
    for (int w = 0; w < NW; ++w)
      for (int64_t si = w; si < sl.n; si += NW) ++dealt;
    CHECK(dealt == sl.n);
    for (int c = 0; c < 32; ++c) {
      const F32mCol x = f32m_column(phase1, c, gsel, hsel, d.L, d.blk, d.anc, q_tokens, d.G,
                                    kv_len, lo, hi);
      if (!x.valid) continue;
      CHECK(x.head >= 0 && x.head < d.Hq && x.head / d.G == kvh);
      // the column's keys: the method's key set, inside the wave's loaded range
      if (phase1) {
        const int64_t i = x.row / d.blk;
        CHECK(x.hiA == (i > 0 ? d.anc : 0) && x.loB == i * d.blk && x.hiB == x.row + 1);
      } else {
        const int64_t pos = kv_len - n_query + x.row;
        CHECK(x.hiA == 0 && x.loB == lo && x.hiB == (hi < pos + 1 ? hi : pos + 1));
      }
      CHECK(x.hiA <= kA);
      if (x.hiB > x.loB) CHECK(x.loB >= kB0 && x.hiB <= kB1);
      outs.mark(phase1 ? (((int64_t)s * d.L + x.row) * d.Hq + x.head)
                       : ((((int64_t)s * n_query + x.row) * d.Hq + x.head) * p->n_split + sigma));
    }
  }
  CHECK(outs.dup == 0 && outs.set == outs.n);
}

static void replay_phase2(const Dims& d, int64_t kv_len, int64_t n_query, int64_t* count) {
  CHECK(validate_phase2(d, kv_len, n_query) == STAR_OK);
  const Plan p = make_plan(d, kv_len, n_query);
  if (d.dtype != STAR_BF16) {
    replay_f32m(d, false, &p, kv_len, n_query);
    ++*count;
    return;
  }
  if (!p.narrow) replay_wide2(d, p, kv_len, n_query);
  else if (p.balanced) replay_decode(d, p, kv_len, n_query);
  else replay_narrow(d, p, kv_len, n_query);
  ++*count;
}

int main() {
  char name[128];
  long long B, Hq, Hkv, D, L, blk, anc, Tq, Td, dt;
  int shapes = 0;
  while (std::scanf("%127s %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", name, &B, &Hq, &Hkv,
                    &D, &L, &blk, &anc, &Tq, &Td, &dt) == 11) {
    g_name = name;
    star_attn_desc x{};
    x.batch = (int32_t)B;
    x.n_q_heads = (int32_t)Hq;
    x.n_kv_heads = (int32_t)Hkv;
    x.head_dim = (int32_t)D;
    x.ctx_len = L;
    x.block_len = blk;
    x.anchor_len = anc;
    x.tail_cap = Tq + Td;
    x.dtype = (int32_t)dt;
    x.softmax_scale = 0.0f;
    Dims d;
    CHECK(validate_desc(&x, &d) == STAR_OK);
    if (g_fail) break;
    std::printf("%s\n", name);
    if (d.dtype == STAR_BF16) replay_phase1(d);
    else replay_f32m(d, true, nullptr, 0, 0);
    // the query step, then decode steps: first, second, a middle one, last
    int64_t n2 = 0;
    replay_phase2(d, L + Tq, Tq, &n2);
    const long long steps[4] = {0, 1, Td / 2, Td - 1};
    for (long long t : steps)
      if (t >= 0 && t < Td) replay_phase2(d, L + Tq + t + 1, 1, &n2);
    std::printf("  phase 2: %lld launches replayed\n", (long long)n2);
    ++shapes;
    std::fflush(stdout);
  }
  if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
  else std::printf("coverage: all checks passed (%d shapes)\n", shapes);
  return g_fail || shapes == 0 ? 1 : 0;
}
