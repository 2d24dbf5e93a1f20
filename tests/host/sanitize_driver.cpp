// Host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Links csrc/star_host.cpp (validation, the phase-2 split planner, the
// extern "C" entry points) against stub launchers that count calls instead of
// launching kernels, then drives every entry point: each validation failure
// (no launcher may run), valid calls on fake pointers (exactly one launch
// sequence), and the planner on thousands of seeded random shapes, checking
// that the splits cover [0, kv_len) once, in order, each inside one host.
// Built and run by tests/test_host_sanitizers.py; no GPU is involved.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "star_internal.hpp"

namespace star {
static int g_launches = 0;
int launch_kv_write(const Dims&, void*, void*, int64_t, const void*, const void*, int64_t, void*,
                    const int32_t*, int32_t, const float*, const float*) {
  ++g_launches;
  return STAR_OK;
}
int launch_phase1(const Dims&, const void*, const void*, const void*, void*, void*, const float*,
                  const float*, int) {
  ++g_launches;
  return STAR_OK;
}
int launch_phase2_partial(const Dims&, const Plan&, const void*, const void*, int64_t,
                          const void*, int64_t, float*, float*, void*, const int32_t*, int32_t) {
  ++g_launches;
  return STAR_OK;
}
int launch_decode_step(const Dims&, const Plan&, void*, void*, int64_t, const void*, const void*,
                       const void*, int64_t, float*, float*, void*, int32_t, float*, void*,
                       const int32_t*, int32_t) {
  ++g_launches;
  return STAR_OK;
}
int launch_lse_merge(const Dims&, int64_t, int32_t, const float*, const float*, void*, int32_t,
                     float*, void*) {
  ++g_launches;
  return STAR_OK;
}
static char g_scratch[64];
int scratch_address(void** ptr) {
  *ptr = g_scratch;  // a fake device address: the stub launchers never touch it
  return STAR_OK;
}
}  // namespace star

static int g_fail = 0;
static int64_t g_splits = 0;  // splits checked
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                   \
    }                                                             \
  } while (0)

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int64_t uniform(int64_t lo, int64_t hi) {  // [lo, hi]
  return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}

static star_attn_desc make(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t L, int64_t b,
                           int64_t a, int64_t cap, int32_t dt) {
  star_attn_desc x;
  x.batch = B;
  x.n_q_heads = Hq;
  x.n_kv_heads = Hkv;
  x.head_dim = d;
  x.ctx_len = L;
  x.block_len = b;
  x.anchor_len = a;
  x.tail_cap = cap;
  x.dtype = dt;
  x.softmax_scale = 0.0f;
  return x;
}

// every split of the plan: contiguous, in order, covering [0, kv_len), each
// inside one host (a context block, or the tail)
static void check_plan(const star_attn_desc& d, int64_t kv_len, int64_t nq) {
  int32_t n = -1;
  CHECK(star_attn_phase2_plan(&d, kv_len, nq, &n) == STAR_OK);
  CHECK(n >= 1);
  const int64_t nb = (d.ctx_len + d.block_len - 1) / d.block_len;
  int64_t last = 0;
  for (int32_t s = 0; s < n; ++s) {
    int64_t lo = -1, hi = -1;
    int32_t host = -1;
    CHECK(star_attn_phase2_split_range(&d, kv_len, nq, s, &lo, &hi, &host) == STAR_OK);
    CHECK(0 <= lo && lo <= hi && hi <= kv_len);
    ++g_splits;
    if (lo == hi) continue;
    CHECK(lo == last);
    last = hi;
    if (host < nb) {
      CHECK(host >= 0 && host * d.block_len <= lo);
      const int64_t end = (host + 1) * d.block_len < d.ctx_len ? (host + 1) * d.block_len
                                                                : d.ctx_len;
      CHECK(hi <= end);
    } else {
      CHECK(host == nb && lo >= d.ctx_len);
    }
  }
  CHECK(last == kv_len);
  int64_t lo, hi;
  int32_t host;
  CHECK(star_attn_phase2_split_range(&d, kv_len, nq, n, &lo, &hi, &host) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase2_split_range(&d, kv_len, nq, -1, &lo, &hi, &host) == STAR_ERR_SHAPE);
}

int main() {
  using star::g_launches;
  char buf[64];
  void* P = buf;  // a fake device pointer: the stubs never touch it
  float* F = (float*)buf;
  const int32_t table[4] = {0, 1, 2, 3};

  for (int s = -6; s <= 1; ++s) CHECK(star_attn_strerror(s) != nullptr);
  CHECK(star_attn_abi_version() >= 1);

  // ---- validation failures launch nothing
  const star_attn_desc ok = make(1, 8, 2, 128, 1000, 256, 100, 40, STAR_BF16);
  star_attn_desc bad[8] = {ok, ok, ok, ok, ok, ok, ok, ok};
  bad[0].n_q_heads = 6;  bad[0].n_kv_heads = 4;  // Hq % Hkv
  bad[1].anchor_len = 300;                       // a > b
  bad[2].head_dim = 96;                          // unsupported
  bad[3].dtype = 7;                              // dtype
  bad[4].batch = 0;
  bad[5].ctx_len = 0;
  bad[6].tail_cap = -1;
  bad[7].softmax_scale = -1.0f;
  int before = g_launches;
  for (const star_attn_desc& b : bad) {
    int32_t n;
    CHECK(star_kv_cache_bytes(&b) == 0);
    CHECK(star_kv_page_bytes(&b) == 0);
    CHECK(star_kv_write(&b, P, P, 0, P, P, 1, nullptr) != STAR_OK);
    CHECK(star_attn_phase1(&b, P, P, P, P, nullptr) != STAR_OK);
    CHECK(star_attn_phase2_plan(&b, 1001, 1, &n) != STAR_OK);
    CHECK(star_attn_phase2_partial(&b, P, P, 1001, P, 1, F, F, nullptr) != STAR_OK);
    CHECK(star_attn_lse_merge(&b, 1, 3, F, F, P, STAR_BF16, nullptr, nullptr) != STAR_OK);
    CHECK(star_attn_decode_step(&b, P, P, 1001, P, P, P, 1, F, F, P, STAR_BF16, nullptr,
                                nullptr) != STAR_OK);
  }
  CHECK(star_kv_cache_bytes(nullptr) == 0);
  CHECK(star_attn_phase1(nullptr, P, P, P, P, nullptr) == STAR_ERR_INVALID_ARG);
  // argument checks on a valid descriptor
  CHECK(star_kv_write(&ok, nullptr, P, 0, P, P, 1, nullptr) == STAR_ERR_INVALID_ARG);
  CHECK(star_kv_write(&ok, P, P, 0, P, P, 0, nullptr) == STAR_ERR_INVALID_ARG);
  CHECK(star_kv_write(&ok, P, P, 1000, P, P, 41, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_kv_write(&ok, P, P, -1, P, P, 1, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase1(&ok, P, nullptr, P, P, nullptr) == STAR_ERR_INVALID_ARG);
  CHECK(star_attn_phase2_partial(&ok, P, P, 1000, P, 1, F, F, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase2_partial(&ok, P, P, 1041, P, 1, F, F, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase2_partial(&ok, P, P, 1005, P, 6, F, F, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase2_partial(&ok, P, P, 1005, P, 1, nullptr, F, nullptr) ==
        STAR_ERR_INVALID_ARG);
  CHECK(star_attn_lse_merge(&ok, 1, 3, F, F, P, 5, nullptr, nullptr) == STAR_ERR_DTYPE);
  CHECK(star_attn_lse_merge(&ok, 41, 3, F, F, P, STAR_BF16, nullptr, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_lse_merge(&ok, 1, 0, F, F, P, STAR_BF16, nullptr, nullptr) ==
        STAR_ERR_INVALID_ARG);
  CHECK(star_attn_decode_step(&ok, P, P, 1005, P, P, P, 1, F, F, P, 9, nullptr, nullptr) ==
        STAR_ERR_DTYPE);
  const int32_t need = (int32_t)((1000 + 40 + 63) / 64);
  CHECK(star_kv_write_paged(&ok, P, P, nullptr, need, 0, P, P, 1, nullptr) ==
        STAR_ERR_INVALID_ARG);
  CHECK(star_kv_write_paged(&ok, P, P, table, need - 1, 0, P, P, 1, nullptr) == STAR_ERR_SHAPE);
  CHECK(star_attn_phase2_partial_paged(&ok, P, P, table, need - 1, 1005, P, 1, F, F, nullptr) ==
        STAR_ERR_SHAPE);
  CHECK(star_attn_decode_step_paged(&ok, P, P, table, need - 1, 1005, P, P, P, 1, F, F, P,
                                    STAR_BF16, nullptr, nullptr) == STAR_ERR_SHAPE);
  star_rope r{F, F, 1040, 0};
  CHECK(star_kv_write_rope(&ok, P, P, 0, P, P, 1, nullptr, nullptr) == STAR_ERR_INVALID_ARG);
  r.n_pos = 1039;
  CHECK(star_kv_write_rope(&ok, P, P, 0, P, P, 1, &r, nullptr) == STAR_ERR_SHAPE);
  r.n_pos = 1040;
  r.anchor_mode = 2;
  CHECK(star_attn_phase1_rope(&ok, P, P, P, &r, P, nullptr) == STAR_ERR_INVALID_ARG);
  CHECK(g_launches == before);

  // ---- 32-bit block and split indices: a block count past INT32_MAX is refused
  for (const int64_t L : {((int64_t)1 << 32) + 5, ((int64_t)1 << 31) + 1}) {
    const star_attn_desc big = make(1, 1, 1, 128, L, 1, 1, 8, STAR_BF16);
    int32_t n = -1;
    before = g_launches;
    CHECK(star_kv_cache_bytes(&big) == 0);
    CHECK(star_attn_phase1(&big, P, P, P, P, nullptr) == STAR_ERR_SHAPE);
    CHECK(star_attn_phase2_plan(&big, L + 1, 1, &n) == STAR_ERR_SHAPE && n == -1);
    CHECK(star_attn_decode_step(&big, P, P, L + 1, P, P, P, 1, F, F, P, STAR_BF16, nullptr,
                                nullptr) == STAR_ERR_SHAPE);
    CHECK(g_launches == before);
  }
  // ---- every grid of a multi-launch call is checked before the first launch:
  // 2^23 query heads, GQA 4:1, 8 query rows: the fused append + partials fit
  // one grid, the merge (2^26 rows) does not, so nothing may be launched
  {
    const star_attn_desc wide = make(1, 1 << 23, 1 << 21, 128, 128, 128, 128, 16, STAR_BF16);
    int32_t n = -1;
    CHECK(star_attn_phase2_plan(&wide, 136, 8, &n) == STAR_OK && n >= 1);
    before = g_launches;
    CHECK(star_attn_decode_step(&wide, P, P, 136, P, P, P, 8, F, F, P, STAR_BF16, nullptr,
                                nullptr) == STAR_ERR_SHAPE);
    CHECK(star_attn_decode_step_paged(&wide, P, P, table, 4, 136, P, P, P, 8, F, F, P, STAR_BF16,
                                      nullptr, nullptr) == STAR_ERR_SHAPE);
    CHECK(star_attn_lse_merge(&wide, 8, n, F, F, P, STAR_BF16, nullptr, nullptr) ==
          STAR_ERR_SHAPE);
    // fp32: three launches (append, partials, merge), the merge too large
    const star_attn_desc wide32 = make(1, 1 << 23, 1 << 21, 64, 128, 128, 128, 16, STAR_F32);
    CHECK(star_attn_decode_step(&wide32, P, P, 136, P, P, P, 8, F, F, P, STAR_F32, nullptr,
                                nullptr) == STAR_ERR_SHAPE);
    CHECK(g_launches == before);
    // one query row: every grid fits, the call launches
    CHECK(star_attn_decode_step(&wide, P, P, 129, P, P, P, 1, F, F, P, STAR_BF16, nullptr,
                                nullptr) == STAR_OK);
    CHECK(g_launches > before);
  }

  // ---- the no-allocation decode step: same checks, plus the scratch size
  {
    before = g_launches;
    CHECK(star_attn_decode_step_noalloc(&ok, P, P, 1005, P, P, P, 1, P, 9, nullptr, nullptr) ==
          STAR_ERR_DTYPE);
    CHECK(star_attn_decode_step_noalloc(&ok, P, P, 1005, nullptr, P, P, 1, P, STAR_BF16, nullptr,
                                        nullptr) == STAR_ERR_INVALID_ARG);
    CHECK(star_attn_decode_step_noalloc(&ok, P, P, 1000, P, P, P, 1, P, STAR_BF16, nullptr,
                                        nullptr) == STAR_ERR_SHAPE);
    // 256 query rows x 64 heads x n_split partials of 129 floats: beyond 16 MiB
    const star_attn_desc big = make(1, 64, 8, 128, 131072, 16384, 16384, 512, STAR_BF16);
    int32_t n = 0;
    CHECK(star_attn_phase2_plan(&big, 131072 + 256, 256, &n) == STAR_OK);
    CHECK((int64_t)256 * 64 * n * 129 * 4 > (int64_t)STAR_NOALLOC_SCRATCH_BYTES);
    CHECK(star_attn_decode_step_noalloc(&big, P, P, 131072 + 256, P, P, P, 256, P, STAR_BF16,
                                        nullptr, nullptr) == STAR_ERR_SHAPE);
    CHECK(g_launches == before);
    CHECK(star_attn_decode_step_noalloc(&ok, P, P, 1005, P, P, P, 1, P, STAR_BF16, nullptr,
                                        nullptr) == STAR_OK);
    CHECK(star_attn_decode_step_noalloc(&big, P, P, 131072 + 1, P, P, P, 1, P, STAR_BF16, nullptr,
                                        nullptr) == STAR_OK);
    CHECK(g_launches > before);
  }

  // ---- valid calls launch (the stubs count)
  r.anchor_mode = 1;
  before = g_launches;
  CHECK(star_kv_write(&ok, P, P, 0, P, P, 1000, nullptr) == STAR_OK);
  CHECK(star_attn_phase1(&ok, P, P, P, P, nullptr) == STAR_OK);
  CHECK(star_attn_phase2_partial(&ok, P, P, 1008, P, 8, F, F, nullptr) == STAR_OK);
  CHECK(star_attn_lse_merge(&ok, 8, 5, F, F, P, STAR_F32, F, nullptr) == STAR_OK);
  CHECK(star_attn_decode_step(&ok, P, P, 1009, P, P, P, 1, F, F, P, STAR_BF16, nullptr,
                              nullptr) == STAR_OK);
  CHECK(star_kv_write_rope(&ok, P, P, 0, P, P, 1000, &r, nullptr) == STAR_OK);
  CHECK(star_attn_phase1_rope(&ok, P, P, P, &r, P, nullptr) == STAR_OK);
  CHECK(g_launches > before);

  // ---- the planner on seeded random shapes (both dtypes, narrow and wide)
  for (int it = 0; it < 2000; ++it) {
    const int32_t Hkv = (int32_t)uniform(1, 8), G = (int32_t)uniform(1, 8);
    const int64_t L = uniform(1, it % 40 == 0 ? 300000 : 5000);
    const int64_t b = uniform(1, L), a = uniform(1, b), cap = uniform(1, 3000);
    const star_attn_desc d = make((int32_t)uniform(1, 4), Hkv * G, Hkv, it % 3 ? 128 : 64, L,
                                  b, a, cap, it % 5 ? STAR_BF16 : STAR_F32);
    CHECK(star_kv_cache_bytes(&d) > 0);
    const int64_t kv_len = L + uniform(1, cap);
    check_plan(d, kv_len, 1);
    check_plan(d, kv_len, uniform(1, kv_len - L));
  }
  // the scope-table shapes at their query and decode steps
  const star_attn_desc big[3] = {make(1, 32, 8, 128, 131072, 16384, 16384, 320, STAR_BF16),
                                 make(1, 32, 8, 128, 1048576, 32768, 32768, 96, STAR_BF16),
                                 make(4, 64, 8, 128, 262144, 32768, 32768, 256, STAR_BF16)};
  for (const star_attn_desc& d : big) {
    check_plan(d, d.ctx_len + 64, 64);
    check_plan(d, d.ctx_len + 65, 1);
    check_plan(d, d.ctx_len + d.tail_cap, 1);
  }
  if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
  else std::printf("host runtime: all checks passed (%lld splits)\n", (long long)g_splits);
  return g_fail ? 1 : 0;
}
