// HIP kernels of libstarattn for gfx950 (CDNA4, 64-wide wavefronts).
//
//   kv_write_kernel     token-major K/V rows -> cache rows (K row-major, V as
//                       transposed 64-row tiles)
//   attn_wide_kernel    flash-style bf16 MFMA tile loop shared by phase 1
//                       (anchor pass + local causal pass, normalised bf16
//                       output) and by phase-2 partials with many query rows
//   attn_wide_short_kernel  the same phase-2 loop for a query tile at most
//                       half full: the waves without live rows only load
//                       tiles and meet barriers
//   attn_decode_kernel  split-KV decode partials (<= 32 query columns), balanced
//                       plan: one cache range per wave, no barriers
//   attn_narrow_kernel  the same for the blockwise plan (blocks shorter than a
//                       balanced range)
//   attn_f32m_kernel    fp32 path on the matrix cores (v_mfma_f32_32x32x2_f32)
//                       for phase 1 (with or without a rotary embedding) and
//                       the phase-2 partials
//   lse_merge_kernel    exact softmax renormalisation of the partials (one
//                       workgroup per output row; lse_merge_rows_kernel: one
//                       wave per row, for many rows)
//
// Method: Star Attention (hotaipapers.com summary page, podcast transcript,
// Phase 1 and Phase 2 descriptions; paperhub.cn rebuttal, reply to reviewer
// EMsM point 5). See include/star_attn.h for the exact definitions.
//
// MFMA formulation. Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: the A operand is a 32-key slice of the K tile
// (from LDS), the B operand is 32 query columns (registers, loaded once).
// The accumulator then holds, per lane, one query column and 16 keys, so the
// softmax max/sum over keys is lane-local plus one exchange with lane ^ 32.
// The same registers, rounded to bf16, are the B operand of O^T += V^T P^T,
// whose A operand is read from the transposed V tile. Key slots of the K tile
// are permuted (bits 2 and 3 of the slot swapped) so that each lane's
// accumulator keys are 8 consecutive keys, i.e. one 16-byte read of V^T.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "star_internal.hpp"

namespace star {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kMinit = -1.0e30f;  // running-max start: finite, below any score

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}


// K-tile slot -> key offset inside a 32-key slice (bits 2 and 3 swapped).
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
// Key (0..31 inside a slice) held in accumulator element i by lane half g.
__device__ __forceinline__ int acc_key(int i, int g) { return ((i >> 3) << 4) + (g << 3) + (i & 7); }

// LDS byte offset of logical 16-byte chunk c of K slot `slot` (XOR swizzle).
template <int D>
__device__ __forceinline__ uint32_t k_off(int slot, int c) {
  return (uint32_t)(slot * (D * 2) + ((c ^ (slot & (D / 8 - 1))) << 4));
}
// LDS byte offset of key chunk kc (8 keys) of row e of a transposed V tile.
// The XOR with bits 1..3 of e spreads the 16 lanes of one LDS cycle (rows
// e .. e+15, same kc) over all 64 banks.
__device__ __forceinline__ int v_swz(int e) { return (e >> 1) & 7; }
__device__ __forceinline__ uint32_t v_off(int e, int kc) {
  return (uint32_t)(e * 128 + ((kc ^ v_swz(e)) << 4));
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 lds16(const char* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void sts16(char* p, u32x4 v) { *(u32x4*)p = v; }

// Zero the bf16 elements of an 8-key chunk whose key lies outside [lo, hi).
__device__ __forceinline__ u32x4 mask_chunk(u32x4 x, int64_t k0, int64_t lo, int64_t hi) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int64_t ka = k0 + 2 * w, kb = ka + 1;
    uint32_t m = 0;
    if (ka >= lo && ka < hi) m |= 0x0000FFFFu;
    if (kb >= lo && kb < hi) m |= 0xFFFF0000u;
    x[w] &= m;
  }
  return x;
}

// Load one 16-byte chunk of a transposed V tile, zeroing keys outside [lo, hi).
__device__ __forceinline__ u32x4 load_v_chunk(const uint16_t* p, int64_t k0, int64_t lo,
                                              int64_t hi) {
  if (k0 >= lo && k0 + 8 <= hi) return ld16(p);
  if (k0 + 8 <= lo || k0 >= hi) return u32x4{0, 0, 0, 0};
  return mask_chunk(ld16(p), k0, lo, hi);
}

// ---- cache addressing ---------------------------------------------------------
//
// Tile t of sequence s and kv head g (cache rows [64t, 64t + 64)) begins at
// the same element offset in the K and in the V buffer: a K tile ([64][D],
// rows) and a transposed V tile ([D][64]) both hold 64 * D elements.
// Contiguous cache: the R / 64 tiles of (s, g) follow each other. Paged
// cache: tile t of sequence s lives in page table[s][t]; a page holds that
// tile for every kv head, kv head g at element (page * Hkv + g) * 64 * D.
struct PageMap {
  const int32_t* table;  // [B][maxp] page ids; null: contiguous cache
  int32_t maxp;
};

template <bool PAGED, int D>
__device__ __forceinline__ int64_t tile_elem(const PageMap& pm, int64_t rows, int Hkv, int s, int g,
                                             int64_t t) {
  if constexpr (PAGED) return ((int64_t)pm.table[(int64_t)s * pm.maxp + t] * Hkv + g) * (64 * D);
  else return (((int64_t)s * Hkv + g) * rows + 64 * t) * D;
}

// The same for a tile index that is uniform across the wave. The table is
// read-only while a kernel runs, so it is read through the constant address
// space: a uniform address then gives a scalar load, which the direct-to-LDS
// loads' vmcnt accounting never sees (a vector load would need a vmcnt wait
// that drains them).
typedef const __attribute__((address_space(4))) int32_t* const_table_ptr;

// Page id of tile t of sequence s (t wave-uniform), by a scalar load.
__device__ __forceinline__ int32_t page_u(const PageMap& pm, int s, int64_t t) {
  const uint64_t ad = (uint64_t)(uintptr_t)(pm.table + ((int64_t)s * pm.maxp + t));
  const uint32_t alo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ad);
  const uint32_t ahi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ad >> 32));
  return *(const_table_ptr)(uintptr_t)(((uint64_t)ahi << 32) | (uint64_t)alo);
}
template <bool PAGED, int D>
__device__ __forceinline__ int64_t tile_elem_u(const PageMap& pm, int64_t rows, int Hkv, int s,
                                               int g, int64_t t) {
  if constexpr (PAGED) {
    return ((int64_t)page_u(pm, s, t) * Hkv + g) * (64 * D);
  } else {
    return tile_elem<false, D>(pm, rows, Hkv, s, g, t);
  }
}

// ---- rotary position embedding ---------------------------------------------
//
// Half-split pairing: element e < D/2 of a head vector turns together with
// element e + D/2 by the angle whose cosine and sine are entry e of the
// table row of the position (fp32 tables [n_pos][D/2]):
//   y_e = x_e c - x_{e+D/2} s,   y_{e+D/2} = x_{e+D/2} c + x_e s.
// fp32 arithmetic with every product and sum rounded on its own (no fused
// multiply-add), then, for bf16 data, one round to nearest even.
enum { kRopeNone = 0, kRopeOriginal = 1, kRopeAdjacent = 2 };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float rope_a(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  return x * c - y * s;
}
__device__ __forceinline__ float rope_b(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  return y * c + x * s;
}

// Two 16-byte chunks of bf16 (8 elements each): lo holds elements e .. e+7,
// hi the elements e + D/2 ..; cr / sr point at table entries e .. e+7.
__device__ __forceinline__ void rope_bf16x8(u32x4& lo, u32x4& hi, const float* cr,
                                            const float* sr) {
  const float4 c0 = *(const float4*)cr, c1 = *(const float4*)(cr + 4);
  const float4 s0 = *(const float4*)sr, s1 = *(const float4*)(sr + 4);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  u32x4 nl, nh;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x0 = bf16_lo(lo[w]), x1 = bf16_hi(lo[w]);
    const float y0 = bf16_lo(hi[w]), y1 = bf16_hi(hi[w]);
    nl[w] = pack_bf16(rope_a(x0, y0, c[2 * w], sn[2 * w]), rope_a(x1, y1, c[2 * w + 1], sn[2 * w + 1]));
    nh[w] = pack_bf16(rope_b(x0, y0, c[2 * w], sn[2 * w]), rope_b(x1, y1, c[2 * w + 1], sn[2 * w + 1]));
  }
  lo = nl;
  hi = nh;
}

// The same for four fp32 elements per chunk (no rounding to bf16).
__device__ __forceinline__ void rope_f32x4(u32x4& lo, u32x4& hi, const float* cr, const float* sr) {
  const float4 c = *(const float4*)cr, sn = *(const float4*)sr;
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
  u32x4 nl, nh;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x = __uint_as_float(lo[w]), y = __uint_as_float(hi[w]);
    nl[w] = __float_as_uint(rope_a(x, y, cc[w], ss[w]));
    nh[w] = __float_as_uint(rope_b(x, y, cc[w], ss[w]));
  }
  lo = nl;
  hi = nh;
}

// ---------------------------------------------------------------------------
// kv_write
// ---------------------------------------------------------------------------
struct KvArgs {
  void* kc;
  void* vc;
  const void* ks;
  const void* vs;
  const float* rope_cos;  // ROPE: K rows rotated at their cache row
  const float* rope_sin;
  PageMap pm;
  int64_t pos0, n_tok, rows, t0;
  int32_t Hkv, nt;
};

template <typename T, int D, bool PAGED, bool ROPE>
__global__ __launch_bounds__(256) void kv_write_kernel(const KvArgs a) {
  constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / VEC;              // chunks per row
  __shared__ __attribute__((aligned(16))) T vsm[64][D + VEC];
  const int tid = threadIdx.x;
  const int64_t tile = a.t0 + blockIdx.x % a.nt;
  const int sg = blockIdx.x / a.nt;
  const int g = sg % a.Hkv, s = sg / a.Hkv;
  const int64_t r0 = tile * 64;
  const int64_t r_lo = a.pos0 > r0 ? a.pos0 : r0;
  const int64_t r_hi = (a.pos0 + a.n_tok) < (r0 + 64) ? (a.pos0 + a.n_tok) : (r0 + 64);
  // this tile's first element in the K and the V buffer
  const int64_t tb = tile_elem<PAGED, D>(a.pm, a.rows, a.Hkv, s, g, tile);
  T* kc = (T*)a.kc;
  T* vc = (T*)a.vc;
  const T* ks = (const T*)a.ks;
  const T* vs = (const T*)a.vs;
  if constexpr (ROPE) {
    // K: chunk c < CPR/2 and its partner chunk c + CPR/2, rotated at row r
    constexpr int HC = CPR / 2;
    for (int u = tid; u < 64 * HC; u += 256) {
      const int rr = u / HC, c = u % HC;
      const int64_t r = r0 + rr;
      if (r >= r_lo && r < r_hi) {
        const int64_t src = (((int64_t)s * a.n_tok + (r - a.pos0)) * a.Hkv + g) * D + c * VEC;
        u32x4 lo = *(const u32x4*)(ks + src), hi = *(const u32x4*)(ks + src + D / 2);
        const float* cr = a.rope_cos + r * (D / 2) + c * VEC;
        const float* sr = a.rope_sin + r * (D / 2) + c * VEC;
        if constexpr (sizeof(T) == 2) rope_bf16x8(lo, hi, cr, sr);
        else rope_f32x4(lo, hi, cr, sr);
        *(u32x4*)(kc + tb + rr * D + c * VEC) = lo;
        *(u32x4*)(kc + tb + rr * D + c * VEC + D / 2) = hi;
      }
    }
    for (int u = tid; u < 64 * CPR; u += 256) {
      const int rr = u / CPR, c = u % CPR;
      const int64_t r = r0 + rr;
      if (r >= r_lo && r < r_hi) {
        const int64_t src = (((int64_t)s * a.n_tok + (r - a.pos0)) * a.Hkv + g) * D + c * VEC;
        *(u32x4*)(&vsm[rr][c * VEC]) = *(const u32x4*)(vs + src);
      }
    }
  } else {
    for (int u = tid; u < 64 * CPR; u += 256) {
      const int rr = u / CPR, c = u % CPR;
      const int64_t r = r0 + rr;
      if (r >= r_lo && r < r_hi) {
        const int64_t src = (((int64_t)s * a.n_tok + (r - a.pos0)) * a.Hkv + g) * D + c * VEC;
        *(u32x4*)(kc + tb + rr * D + c * VEC) = *(const u32x4*)(ks + src);
        *(u32x4*)(&vsm[rr][c * VEC]) = *(const u32x4*)(vs + src);
      }
    }
  }
  __syncthreads();
  T* vt = vc + tb;  // transposed tile: element (e, kk) at e*64 + kk
  if (r_lo == r0 && r_hi == r0 + 64) {
    constexpr int KC = 64 / VEC;
    for (int u = tid; u < D * KC; u += 256) {
      const int e = u / KC, kc0 = (u % KC) * VEC;
      T tmp[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) tmp[j] = vsm[kc0 + j][e];
      *(u32x4*)(vt + e * 64 + kc0) = *(const u32x4*)tmp;
    }
  } else {
    for (int u = tid; u < D * 64; u += 256) {
      const int e = u / 64, kk = u % 64;
      const int64_t r = r0 + kk;
      if (r >= r_lo && r < r_hi) vt[e * 64 + kk] = vsm[kk][e];
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel: NW waves x (32 * QT) query columns share 64-key K / V^T tiles
// in LDS. Columns are (query row, head) pairs of one kv head.
// ---------------------------------------------------------------------------
struct WideArgs {
  const uint16_t* k;  // cache K (row-major rows)
  const uint16_t* v;  // cache V (transposed 64-row tiles)
  const uint16_t* q;  // [B][q_tokens][Hq][D]
  uint16_t* o;        // phase 1: [B][L][Hq][D]
  float* o_part;      // phase 2: [B][n_query][Hq][n_split][D]
  float* lse_part;    // phase 2: [B][n_query][Hq][n_split]
  int64_t rows;       // cache rows per (seq, kv head)
  int64_t q_tokens;   // tokens per sequence in q (ctx_len or n_query)
  int64_t L, blk, anc, kv_len;
  int64_t blk_len, tail_len;  // split plan
  int32_t per_block, n_split, n_blocks;
  int32_t Hq, Hkv, G, HW, HQ, NG, NRT;  // NRT: row tiles (phase 1) / query tiles (phase 2)
  int32_t BM;                           // rows per workgroup = 64 * (4 / HW)
  float scale, c2;                      // softmax scale and scale*log2(e)
  PageMap pm;                           // phase 2 on a paged cache
  const float* rope_cos;                // ROPE (phase 1): tables [n_pos][D/2]
  const float* rope_sin;
};

// max / sum with the lane 32 apart (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- geometry ----------------------------------------------------------------
//
// Interior tiles (all 64 keys visible to every query column of the
// workgroup) are loaded with global_load_lds_dwordx4, which writes lane i's
// 16 bytes at LDS base + 16*i: each lane fetches the global chunk that the
// swizzled LDS layout wants at its slot. Tiles are prefetched two ahead into
// a ring of four stages; the LDS holds the four K tiles, then the four
// transposed V tiles, so every operand read is a per-lane register plus an
// immediate below 64 KB. The loop is software-pipelined per 32-key slice:
// while the softmax of slice u runs on the VALU, the MFMAs of S(u+1) are
// issued, and the row max of S(u+1) overlaps the P.V MFMAs of slice u.
//
// Lazy rescale: the running max m of a column only moves when a slice max
// exceeds it by more than kTau in the exp2 domain, so P <= 2^kTau and the O
// accumulators are rescaled (by exp2((m_old - m_new) * c2)) only then; the
// final O / l uses the same m, so the result is unchanged.
constexpr float kTau = 8.0f;
constexpr int kStages = 4;

typedef __attribute__((address_space(3))) void lds_void;

template <int D, int NW>
struct Geo {
  static constexpr int NT = 64 * NW;             // threads
  static constexpr int CH = D / 8;              // 16-byte chunks per K row
  static constexpr int RB = 2 * D;              // bytes per K row
  static constexpr int KBYTES = 64 * RB;        // K tile
  static constexpr int VBYTES = D * 128;        // transposed V tile (D rows x 64 keys)
  static constexpr int K_AT = 0;                // ring: K tiles of the stages
  static constexpr int V_AT = kStages * KBYTES; //       then V tiles
  static constexpr int RING = kStages * (KBYTES + VBYTES);
  static constexpr int KI = KBYTES / 1024 / NW; // 1-KB DMA instructions per wave, K
  static constexpr int VI = VBYTES / 1024 / NW; // and V
  static constexpr int PER = KI + VI;           // DMA instructions per thread per tile
  static constexpr int SPK = 1024 / RB;         // K slots per KB
  static constexpr int KS = D / 16;             // k-steps over the head dimension
  static constexpr int DT = D / 32;             // 32-row tiles of the output dimension
  static_assert(KI >= 1 && VI >= 1, "tile too small for the wave count");
};

// s_waitcnt vmcnt(N) leaving expcnt / lgkmcnt untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vm_lgk0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
}

// Register-staged tile load for edge tiles: zero for keys outside [lo, hi),
// written into stage 0 of the ring.
template <int D, int NW>
struct EdgeTile {
  using Gm = Geo<D, NW>;
  static constexpr int KPT = 64 * Gm::CH / Gm::NT;
  static constexpr int VPT = D * 8 / Gm::NT;
  u32x4 kr[KPT], vr[VPT];

  // Kt, Vt: the tile holding keys [kbase, kbase + 64)
  __device__ __forceinline__ void load(const uint16_t* Kt, const uint16_t* Vt, int64_t kbase,
                                       int64_t lo, int64_t hi, int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = tid + Gm::NT * i, slot = u / Gm::CH, c = u % Gm::CH;
      const int kk = (slot & 32) + swap23(slot & 31);
      const int64_t key = kbase + kk;
      kr[i] = (key >= lo && key < hi) ? ld16(Kt + kk * D + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + Gm::NT * i, e = u >> 3, kc = u & 7;
      vr[i] = load_v_chunk(Vt + e * 64 + kc * 8, kbase + kc * 8, lo, hi);
    }
  }
  __device__ __forceinline__ void store(char* smem, int tid) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = tid + Gm::NT * i;
      sts16(smem + Gm::K_AT + k_off<D>(u / Gm::CH, u % Gm::CH), kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + Gm::NT * i;
      sts16(smem + Gm::V_AT + v_off(u >> 3, u & 7), vr[i]);
    }
  }
};

// Per-lane constant offsets, computed once per workgroup.
template <int D, int NW>
struct LaneOffsets {
  using Gm = Geo<D, NW>;
  uint32_t kq[Gm::KS];  // K operand, slice 0, k-step ks (bytes inside a K tile)
  uint32_t vq[2][2];    // V operand, [kt][kb], dt = 0 (bytes from the ring start)
  uint32_t kd[Gm::KI];  // DMA: global byte offset of this lane's K chunk in a tile
  uint32_t vd[Gm::VI];  // DMA: global byte offset of this lane's V chunk in a tile

  __device__ __forceinline__ void init(int l32, int g, int w, int lane) {
#pragma unroll
    for (int ks = 0; ks < Gm::KS; ++ks) kq[ks] = k_off<D>(l32, 2 * ks + g);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        vq[kt][kb] = (uint32_t)Gm::V_AT + v_off(l32, 4 * kt + 2 * kb + g);
#pragma unroll
    for (int j = 0; j < Gm::KI; ++j) {
      const int slot = Gm::SPK * (Gm::KI * w + j) + lane / Gm::CH;
      const int c = (lane % Gm::CH) ^ (slot & (Gm::CH - 1));
      kd[j] = (uint32_t)(((slot & 32) + swap23(slot & 31)) * Gm::RB + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < Gm::VI; ++j) {
      const int e = 8 * (Gm::VI * w + j) + (lane >> 3);
      const int kc = (lane & 7) ^ v_swz(e);
      vd[j] = (uint32_t)((e * 64 + 8 * kc) * 2);
    }
  }
};

// One direct-to-LDS load (global_load_lds_dwordx4: lane i's 16 bytes from
// gbase + voff land at LDS lds + 16 i), issued through a minimal asm
// statement rather than the builtin. The compiler then keeps no record of it
// as an LDS write and inserts no drain of the load counter before later LDS
// reads; the caller waits with explicit vmcnt (and lgkmcnt before reusing a
// stage) and a barrier before reading a stage. The asm has no register
// outputs: the data lands in LDS.
//
// The compiler's hazard recognizer does not look inside asm, so the asm
// supplies the wait states itself: an SALU write of M0 needs one before an
// LDS DMA reads it, a VALU write of an SGPR (v_readfirstlane) five before a
// VMEM instruction reads it; s_nop 4 gives five.
//
// NT sets the non-temporal cache policy: for data that one launch reads once
// (the phase-2 stream over the cache), so it does not displace what other
// loads reuse. On MI355X a non-temporal stream also reads HBM faster: 7.1 TB/s
// against 6.0 TB/s for the same 512 MiB stream with the default policy.
template <bool NT = false>
__device__ __forceinline__ void dma16_lds(const char* gbase, uint32_t voff, const char* lds) {
  // the base is wave-uniform: pin it to an SGPR pair for the saddr operand.
  // readfirstlane returns int: go through uint32_t so the low half is
  // zero-extended, not sign-extended into the high half
  const uint64_t gb = (uint64_t)(uintptr_t)gbase;
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gb);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gb >> 32));
  const uint64_t gs = ((uint64_t)ghi << 32) | (uint64_t)glo;
  const uint32_t m0 =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)lds);
  if constexpr (NT)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(gs), "{m0}"(m0)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gs), "{m0}"(m0)
                 : "memory");
}

template <int D, int NW, int ST, bool NT>
__device__ __forceinline__ void dma_stage_asm(char* smem, const char* Kt, const char* Vt,
                                              const LaneOffsets<D, NW>& lo, int w) {
  using Gm = Geo<D, NW>;
#pragma unroll
  for (int j = 0; j < Gm::KI; ++j)
    dma16_lds<NT>(Kt, lo.kd[j], smem + Gm::K_AT + ST * Gm::KBYTES + (Gm::KI * w + j) * 1024);
#pragma unroll
  for (int j = 0; j < Gm::VI; ++j)
    dma16_lds<NT>(Vt, lo.vd[j], smem + Gm::V_AT + ST * Gm::VBYTES + (Gm::VI * w + j) * 1024);
}

// S^T of one 32-key slice KT of stage ST for the QT column tiles.
template <int D, int NW, int QT, int ST, int KT>
__device__ __forceinline__ void qk_slice(const char* smem, const LaneOffsets<D, NW>& lo,
                                         const u32x4 (&q)[QT][Geo<D, NW>::KS], f32x16 (&s)[QT]) {
  using Gm = Geo<D, NW>;
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    const u32x4 kop = lds16(smem + lo.kq[ks] + (Gm::K_AT + ST * Gm::KBYTES + KT * 32 * Gm::RB));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[qt] = mfma_bf16(kop, q[qt][ks], ks == 0 ? f32x16{} : s[qt]);
  }
}

// The first kKA K operands (k-steps) of a slice's QK, read from LDS ahead of
// the chain into registers; qk_ahead runs the chain on them and reads the
// rest as it goes. Holding four ahead takes the LDS latency off the start of
// each half-stage (phase 1 at 128K 1.7% faster, bit-identical); all eight
// ahead spill registers.
constexpr int kKA = 4;

template <int D, int NW, int ST, int KT>
__device__ __forceinline__ void k_ahead(const char* smem, const LaneOffsets<D, NW>& lo,
                                        u32x4 (&kop)[kKA]) {
  using Gm = Geo<D, NW>;
#pragma unroll
  for (int ks = 0; ks < kKA; ++ks)
    kop[ks] = lds16(smem + lo.kq[ks] + (Gm::K_AT + ST * Gm::KBYTES + KT * 32 * Gm::RB));
}

template <int D, int NW, int QT, int ST, int KT>
__device__ __forceinline__ void qk_ahead(const char* smem, const LaneOffsets<D, NW>& lo,
                                         const u32x4 (&kop)[kKA],
                                         const u32x4 (&q)[QT][Geo<D, NW>::KS], f32x16 (&s)[QT]) {
  using Gm = Geo<D, NW>;
  static_assert(Gm::KS >= kKA, "head_dim too small for the operands read ahead");
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks) {
    const u32x4 kv = ks < kKA ? kop[ks]
                              : lds16(smem + lo.kq[ks] + (Gm::K_AT + ST * Gm::KBYTES + KT * 32 * Gm::RB));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[qt] = mfma_bf16(kv, q[qt][ks], ks == 0 ? f32x16{} : s[qt]);
  }
}

// O^T += V^T P^T for one 32-key slice KT of stage ST.
template <int D, int NW, int QT, int ST, int KT>
__device__ __forceinline__ void pv_slice(const char* smem, const LaneOffsets<D, NW>& lo,
                                         const u32x4 (&p)[QT][2], f32x16 (&o)[QT][Geo<D, NW>::DT]) {
  using Gm = Geo<D, NW>;
  // the first half of P (keys 0-15) feeds the first DT MFMAs, so the exps
  // of the second half have that long to land; every O tile still adds
  // half 0 then half 1
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) {
      const u32x4 vop = lds16(smem + lo.vq[KT][kb] + (ST * Gm::VBYTES + dt * 32 * 128));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) o[qt][dt] = mfma_bf16(vop, p[qt][kb], o[qt][dt]);
    }
}

template <int QT>
__device__ __forceinline__ void slice_max3(const f32x16 (&s)[QT], float (&mx)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // a tree of 3-input maxima (v_max3_f32), depth 3
    const auto m3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
    const float x0 = m3(s[qt][0], s[qt][1], s[qt][2]), x1 = m3(s[qt][3], s[qt][4], s[qt][5]);
    const float x2 = m3(s[qt][6], s[qt][7], s[qt][8]), x3 = m3(s[qt][9], s[qt][10], s[qt][11]);
    const float x4 = m3(s[qt][12], s[qt][13], s[qt][14]);
    const float x = fmaxf(m3(x0, x1, x2), m3(x3, x4, s[qt][15]));
    mx[qt] = pair_max(x);
  }
}

// Move the running max (and rescale O, l) when a slice max exceeds it by
// more than kTau; wave-uniform branch, taken rarely.
template <int QT, int DT>
__device__ __forceinline__ void rescale_top(const float (&mx)[QT], float (&m)[QT], float (&l)[QT],
                                            f32x16 (&o)[QT][DT], float c2) {
  bool need = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) need |= (mx[qt] - m[qt]) * c2 > kTau;
  if (__any(need)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float m_new = fmaxf(m[qt], mx[qt]);
      const float al = fast_exp2((m[qt] - m_new) * c2);
      m[qt] = m_new;
      l[qt] *= al;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= al;
    }
  }
}

// exp2 + bf16 pack + row sum of the packed values (v_dot2c_f32_bf16), so l is
// the sum of exactly the weights that enter P.V.
template <int QT>
__device__ __forceinline__ void slice_exp2(const f32x16 (&s)[QT], const float (&m)[QT],
                                           float (&l)[QT], u32x4 (&p)[QT][2], float c2) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float mc = m[qt] * c2;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t w4[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int i = 8 * kb + 2 * h;
        const uint32_t pk = pack_bf16(fast_exp2(fmaf(s[qt][i], c2, -mc)),
                                      fast_exp2(fmaf(s[qt][i + 1], c2, -mc)));
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, rs, false);
        w4[h] = pk;
      }
      p[qt][kb] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
    l[qt] += rs;
  }
}

// A stage of the interior loop for a wave with no live query row: the same
// wait, barrier and tile load as interior_stage, no arithmetic.
template <int D, int NW, int ST, bool NT>
__device__ __forceinline__ void idle_stage(char* smem, const LaneOffsets<D, NW>& lo,
                                           const char* Kt3, const char* Vt3, int w) {
  using Gm = Geo<D, NW>;
  wait_vm_lgk0<Gm::PER>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  dma_stage_asm<D, NW, (ST + 3) & 3, NT>(smem, Kt3, Vt3, lo, w);
}

// One 64-key stage of the software-pipelined interior loop: slice (t,0)
// then slice (t,1); the first QK of the next stage is issued in the second
// half, after the ring barrier and the DMA of tile t + 3. `ka` holds the
// first K operands of half A's QK (stage ST, slice 1), read at the end of the
// previous stage; those of half B's QK (stage ST + 1, slice 0) are read right
// after the barrier, and the stage ends by reading the next stage's half-A
// operands (stage ST + 1 landed before the barrier).
template <int D, int NW, int QT, int ST, bool NT>
__device__ __forceinline__ void interior_stage(char* smem, const LaneOffsets<D, NW>& lo,
                                               const u32x4 (&q)[QT][Geo<D, NW>::KS],
                                               f32x16 (&sc)[QT], float (&mx)[QT], float (&m)[QT],
                                               float (&l)[QT], f32x16 (&o)[QT][Geo<D, NW>::DT],
                                               u32x4 (&ka)[kKA], float c2, const char* Kt3,
                                               const char* Vt3, int w) {
  using Gm = Geo<D, NW>;
  rescale_top<QT, Gm::DT>(mx, m, l, o, c2);
  {
    f32x16 sn[QT];
    u32x4 p[QT][2];
    qk_ahead<D, NW, QT, ST, 1>(smem, lo, ka, q, sn);
    slice_exp2<QT>(sc, m, l, p, c2);
    pv_slice<D, NW, QT, ST, 0>(smem, lo, p, o);
    slice_max3<QT>(sn, mx);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sc[qt] = sn[qt];
  }
  rescale_top<QT, Gm::DT>(mx, m, l, o, c2);
  // tile t + 1 has landed (this wave's loads; the barrier covers the other
  // waves') and every wave's reads of stage ST + 3 (tile t - 1) are complete
  wait_vm_lgk0<Gm::PER>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read moves above the wait
  u32x4 kb[kKA];
  k_ahead<D, NW, (ST + 1) & 3, 0>(smem, lo, kb);
  dma_stage_asm<D, NW, (ST + 3) & 3, NT>(smem, Kt3, Vt3, lo, w);
  {
    f32x16 sn[QT];
    u32x4 p[QT][2];
    qk_ahead<D, NW, QT, (ST + 1) & 3, 0>(smem, lo, kb, q, sn);
    slice_exp2<QT>(sc, m, l, p, c2);
    pv_slice<D, NW, QT, ST, 1>(smem, lo, p, o);
    slice_max3<QT>(sn, mx);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sc[qt] = sn[qt];
  }
  k_ahead<D, NW, (ST + 1) & 3, 1>(smem, lo, ka);
  // keep these reads here, ahead of the next stage's rescale check
  __builtin_amdgcn_sched_barrier(0);
}

// Wave -> columns: wave w owns QT column tiles of 32 (query row, head) pairs.
// The workgroup covers 256 columns: HW heads of one kv head x 64*(4/HW) rows.
// KVNT: the interior K/V tiles are read with the non-temporal policy. Phase 2
// takes it when each split's keys are read by one workgroup; when several
// workgroups read them (query-head sub-groups, query tiles), and in phase 1,
// the default policy lets L2 serve the re-reads.
// SHORT (phase 2): a query tile with at most half its rows live; the waves
// without live rows load their share of every tile and meet every barrier,
// but skip the arithmetic (see wide_wave).
template <int D, int NW, int QT, bool PHASE1, bool PAGED, int ROPE, bool KVNT, bool SHORT>
__device__ __forceinline__ void wide_body(const WideArgs& a, char* smem) {
  static_assert(!(PHASE1 && PAGED), "phase 1 reads the contiguous cache");
  static_assert(!(PHASE1 && KVNT), "phase 1 reuses its tiles through L2");
  static_assert(PHASE1 || ROPE == kRopeNone, "rotary embedding is fused into phase 1");
  static_assert(!(PHASE1 && SHORT), "short query tiles are a phase-2 case");
  static_assert(!SHORT || QT == 1, "short tiles: one 32-column tile per wave");
  using Gm = Geo<D, NW>;
  constexpr int KS = Gm::KS, DT = Gm::DT;
  static_assert(NW * QT == 8, "workgroup covers 256 columns");
  // the wave index is uniform: keep it (and what derives from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // ---- which (group, work item) this workgroup is (XCD-aware order)
  int32_t gidx;
  int64_t work;
  wide_map(blockIdx.x, PHASE1, a.NG, a.HQ, a.NRT, a.n_split, a.n_blocks, &gidx, &work);
  const int hq = gidx % a.HQ, t2 = gidx / a.HQ;
  const int kvh = t2 % a.Hkv, s = t2 / a.Hkv;
  int hw;
  int64_t wrow_off;  // this wave's first query row, from the workgroup's
  wide_wave(w, QT, a.HW, SHORT, &hw, &wrow_off);
  const int head = kvh * a.G + hq * a.HW + hw;

  int64_t row0, row_end, hiA = 0, loB, hiB, pos_off;
  int32_t sigma = 0;
  if (PHASE1) {
    int64_t i, rt;
    phase1_item(work, a.n_blocks, a.NRT, &i, &rt);
    row0 = i * a.blk + rt * a.BM;
    row_end = (i + 1) * a.blk < a.L ? (i + 1) * a.blk : a.L;
    if (row0 >= row_end) return;
    if (i > 0) hiA = a.anc;
    loB = i * a.blk;
    hiB = row0 + a.BM < row_end ? row0 + a.BM : row_end;
    pos_off = 0;
  } else {
    const int64_t qrt = work % a.NRT;
    sigma = (int32_t)(work / a.NRT);
    row0 = qrt * a.BM;
    row_end = a.q_tokens;
    if (row0 >= row_end) return;
    int32_t host;
    split_rows(a.L, a.blk, a.n_blocks, a.per_block, a.blk_len, a.tail_len, a.kv_len, sigma, &loB,
               &hiB, &host);
    pos_off = a.kv_len - a.q_tokens;
  }
  const int64_t wrow0 = row0 + wrow_off;  // this wave's first query row
  const bool idle = SHORT && wrow0 >= row_end;  // no live row: loads and barriers only
  const int64_t head_row0 = ((int64_t)s * a.Hkv + kvh) * a.rows;
  const uint16_t* K = PAGED ? a.k : a.k + head_row0 * D;
  const uint16_t* V = PAGED ? a.v : a.v + head_row0 * D;
  // element offset of this (sequence, kv head)'s tile t from K and from V
  auto tile_at = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem_u<true, D>(a.pm, a.rows, a.Hkv, s, kvh, t);
    else return t * 64 * D;
  };
  const float c2 = a.c2;

  // ---- query operand (B of S^T = K Q^T): column 32*qt + l32, d-chunk 2*ks + g.
  // With a rotary embedding the query is turned at its position id, the
  // context row less `shift`; chunk ks and chunk ks + KS/2 of a lane hold
  // the element pairs (e, e + D/2) that turn together.
  u32x4 qop[QT][KS];
  auto load_q = [&](int64_t shift) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t r = wrow0 + 32 * qt + l32;
      const bool ok = r < row_end;
      const uint16_t* qp = a.q + (((int64_t)s * a.q_tokens + (ok ? r : 0)) * a.Hq + head) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qop[qt][ks] = ok ? ld16(qp + (2 * ks + g) * 8) : u32x4{0, 0, 0, 0};
      if constexpr (ROPE != kRopeNone) {
        const int64_t pos = ok ? r - shift : 0;
        const float* cr = a.rope_cos + pos * (D / 2);
        const float* sr = a.rope_sin + pos * (D / 2);
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks)
          rope_bf16x8(qop[qt][ks], qop[qt][ks + KS / 2], cr + 8 * (2 * ks + g),
                      sr + 8 * (2 * ks + g));
      }
    }
  };
  // adjacent anchor ids (i*b - a + j for anchor row j of block i): rotations
  // compose, so the anchor pass keeps the cached keys and turns the query
  // back by i*b - a instead
  const int64_t q_shift =
      (ROPE == kRopeAdjacent && PHASE1 && hiA > 0) ? (row0 / a.blk) * a.blk - a.anc : 0;
  load_q(q_shift);

  f32x16 oacc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x16{};
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = kMinit;
    l[qt] = 0.0f;
  }

  // ---- tile classes. Range A: anchor [0, hiA), no mask. Range B: [loB, hiB),
  // causal (key <= query position). Interior tiles need no mask at all.
  const TileRuns runs = tile_runs(hiA, loB, hiB, row0 + pos_off);
  const int nAi = (int)runs.nAi;
  const bool a_edge = runs.a_edge != 0;
  const int64_t bf = runs.bf, bl = runs.bl, i0 = runs.i0, i1 = runs.i1;
  const int n_int = nAi + (int)(i1 - i0);
  // interior tiles j0 .. j0 + cnt - 1 (anchor tiles first, then the block's);
  // tile j of the run -> byte offset of its rows (clamped to the last tile)
  auto run_interior = [&](const int j0, const int cnt) {
  auto tile_off = [&](int j) -> int64_t {
    j = j0 + (j < cnt ? j : cnt - 1);
    return tile_at(j < nAi ? (int64_t)j : i0 + (j - nAi)) * 2;
  };
  const int n_int = cnt;
  if (n_int > 0) {
    LaneOffsets<D, NW> lo;
    lo.init(l32, g, w, lane);
    const char* Kc = (const char*)K;
    const char* Vc = (const char*)V;
    dma_stage_asm<D, NW, 0, KVNT>(smem, Kc + tile_off(0), Vc + tile_off(0), lo, w);
    dma_stage_asm<D, NW, 1, KVNT>(smem, Kc + tile_off(1), Vc + tile_off(1), lo, w);
    dma_stage_asm<D, NW, 2, KVNT>(smem, Kc + tile_off(2), Vc + tile_off(2), lo, w);
    wait_vmcnt<2 * Gm::PER>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the wait
    if (idle) {
      // the same waits, barriers and tile loads as interior_stage
      for (int t = 0; t < n_int; t += 4) {
        idle_stage<D, NW, 0, KVNT>(smem, lo, Kc + tile_off(t + 3), Vc + tile_off(t + 3), w);
        if (t + 1 >= n_int) break;
        idle_stage<D, NW, 1, KVNT>(smem, lo, Kc + tile_off(t + 4), Vc + tile_off(t + 4), w);
        if (t + 2 >= n_int) break;
        idle_stage<D, NW, 2, KVNT>(smem, lo, Kc + tile_off(t + 5), Vc + tile_off(t + 5), w);
        if (t + 3 >= n_int) break;
        idle_stage<D, NW, 3, KVNT>(smem, lo, Kc + tile_off(t + 6), Vc + tile_off(t + 6), w);
      }
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      return;
    }
    f32x16 sc[QT];
    float mx[QT];
    qk_slice<D, NW, QT, 0, 0>(smem, lo, qop, sc);
    slice_max3<QT>(sc, mx);
    u32x4 ka[kKA];
    k_ahead<D, NW, 0, 1>(smem, lo, ka);
    for (int t = 0; t < n_int; t += 4) {
      interior_stage<D, NW, QT, 0, KVNT>(smem, lo, qop, sc, mx, m, l, oacc, ka, c2,
                                            Kc + tile_off(t + 3), Vc + tile_off(t + 3), w);
      if (t + 1 >= n_int) break;
      interior_stage<D, NW, QT, 1, KVNT>(smem, lo, qop, sc, mx, m, l, oacc, ka, c2,
                                            Kc + tile_off(t + 4), Vc + tile_off(t + 4), w);
      if (t + 2 >= n_int) break;
      interior_stage<D, NW, QT, 2, KVNT>(smem, lo, qop, sc, mx, m, l, oacc, ka, c2,
                                            Kc + tile_off(t + 5), Vc + tile_off(t + 5), w);
      if (t + 3 >= n_int) break;
      interior_stage<D, NW, QT, 3, KVNT>(smem, lo, qop, sc, mx, m, l, oacc, ka, c2,
                                            Kc + tile_off(t + 6), Vc + tile_off(t + 6), w);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }
  };

  // ---- edge tiles e0 .. e1 - 1 (the anchor's partial tile first, if any):
  // masked, synchronous, staged through registers with zero fill
  const int n_edge = (a_edge ? 1 : 0) + (int)(i0 - bf) + (int)(bl - i1);
  auto run_edges = [&](const int e0, const int e1) {
  if (e1 > e0) {
    LaneOffsets<D, NW> lo;
    lo.init(l32, g, w, lane);
    for (int e = e0; e < e1; ++e) {
      int64_t kbase, klo, khi;
      bool causal;
      int k = e;
      if (a_edge && k == 0) {
        kbase = (int64_t)nAi * 64; klo = 0; khi = hiA; causal = false;
      } else {
        k -= a_edge ? 1 : 0;
        kbase = (k < i0 - bf ? bf + k : i1 + (k - (i0 - bf))) * 64;
        klo = loB; khi = hiB; causal = true;
      }
      EdgeTile<D, NW> et;
      et.load(K + tile_at(kbase / 64), V + tile_at(kbase / 64), kbase, klo, khi, tid);
      et.store(smem, tid);
      block_sync_lds();
      if (!idle)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 sc[QT];
        if (kt == 0) qk_slice<D, NW, QT, 0, 0>(smem, lo, qop, sc);
        else qk_slice<D, NW, QT, 0, 1>(smem, lo, qop, sc);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int64_t pos = wrow0 + 32 * qt + l32 + pos_off;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t key = kbase + 32 * kt + acc_key(i, g);
            if (key < klo || key >= khi || (causal && key > pos)) sc[qt][i] = -INFINITY;
          }
        }
        float mx[QT];
        slice_max3<QT>(sc, mx);
        rescale_top<QT, DT>(mx, m, l, oacc, c2);
        u32x4 p[QT][2];
        slice_exp2<QT>(sc, m, l, p, c2);
        if (kt == 0) pv_slice<D, NW, QT, 0, 0>(smem, lo, p, oacc);
        else pv_slice<D, NW, QT, 0, 1>(smem, lo, p, oacc);
      }
      block_sync_lds();
    }
  }
  };

  if constexpr (ROPE == kRopeAdjacent) {
    // the anchor (interior tiles, then its partial tile) with the turned-back
    // query, then the block with the query at its own position
    run_interior(0, nAi);
    run_edges(0, a_edge ? 1 : 0);
    if (q_shift != 0) load_q(0);
    run_interior(nAi, n_int - nAi);
    run_edges(a_edge ? 1 : 0, n_edge);
  } else {
    run_interior(0, n_int);
    run_edges(0, n_edge);
  }

  // ---- epilogue: accumulator element i of tile dt is dimension 32*dt + 8*(i/4) + 4*g + i%4
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = pair_sum(l[qt]);
    const int64_t r = wrow0 + 32 * qt + l32;
    if (r >= row_end) continue;
    if (PHASE1) {
      const float inv = 1.0f / lt;
      uint16_t* op = a.o + (((int64_t)s * a.L + r) * a.Hq + head) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x16& x = oacc[qt][dt];
          uint2 v2;
          v2.x = pack_bf16(x[4 * j4 + 0] * inv, x[4 * j4 + 1] * inv);
          v2.y = pack_bf16(x[4 * j4 + 2] * inv, x[4 * j4 + 3] * inv);
          *(uint2*)(op + 32 * dt + 8 * j4 + 4 * g) = v2;
        }
    } else {
      const bool any = lt > 0.0f;
      const float inv = any ? 1.0f / lt : 0.0f;
      const int64_t base = (((int64_t)s * a.q_tokens + r) * a.Hq + head) * a.n_split + sigma;
      float* op = a.o_part + base * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x16& x = oacc[qt][dt];
          *(f32x4*)(op + 32 * dt + 8 * j4 + 4 * g) =
              f32x4{x[4 * j4] * inv, x[4 * j4 + 1] * inv, x[4 * j4 + 2] * inv, x[4 * j4 + 3] * inv};
        }
      if (g == 0) a.lse_part[base] = any ? m[qt] * a.scale + logf(lt) : -INFINITY;
    }
  }
}

template <int D, int NW, int QT, bool PHASE1, bool PAGED, int ROPE, bool KVNT>
__global__ __launch_bounds__(64 * NW) void attn_wide_kernel(const WideArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Geo<D, NW>::RING];
  wide_body<D, NW, QT, PHASE1, PAGED, ROPE, KVNT, false>(a, smem);
}

// Phase 2 with a short query tile (wide2_short): the waves that hold no live
// row leave the matrix cores to their SIMD partners.
template <int D, int NW, bool PAGED, bool KVNT>
__global__ __launch_bounds__(64 * NW) void attn_wide_short_kernel(const WideArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Geo<D, NW>::RING];
  wide_body<D, NW, 1, false, PAGED, kRopeNone, KVNT, true>(a, smem);
}

// ---------------------------------------------------------------------------
// Narrow kernel (decode): one 32-column tile of (query, head-in-group) pairs
// per (sequence, kv head, split). Stages of 128 keys; wave w owns keys
// [32w, 32w + 32) of each stage with its own softmax state; the four states
// are merged through LDS at the end.
// ---------------------------------------------------------------------------
struct NarrowArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;  // [B][n_query][Hq][D]
  float* o_part;
  float* lse_part;
  int64_t rows, L, blk, kv_len, n_query;
  int64_t blk_len, tail_len;
  int32_t per_block, n_split, n_blocks;
  int32_t Hq, Hkv, G, NG;
  float scale, c2;
  // decode step (FUSED kernels only): rows appended at kv_len - n_query
  const uint16_t* k_new;  // [B][n_query][Hkv][D]
  const uint16_t* v_new;
  PageMap pm;             // paged cache
};

// Decode ring: kNarrowStages stages, each one 64-key tile laid out as
// [K tile | transposed V tile] (LDS layouts as in the wide kernel).
constexpr int kNarrowStages = 5;
template <int D>
struct NarrowRing {
  using Gm = Geo<D, 4>;
  static constexpr int SB = Gm::KBYTES + Gm::VBYTES;  // bytes per stage
  static constexpr int BYTES = kNarrowStages * SB;
};

// This wave's share of the direct-to-LDS loads of one tile into stage ST.
template <int D, int ST>
__device__ __forceinline__ void dma_stage_narrow(char* smem, const char* Kt, const char* Vt,
                                                 const LaneOffsets<D, 4>& lo, int w) {
  using Gm = Geo<D, 4>;
  char* st = smem + ST * NarrowRing<D>::SB;
  // non-temporal K only: measured 2% faster per decode step than both
#pragma unroll
  for (int j = 0; j < Gm::KI; ++j) dma16_lds<true>(Kt, lo.kd[j], st + (Gm::KI * w + j) * 1024);
#pragma unroll
  for (int j = 0; j < Gm::VI; ++j)
    dma16_lds<false>(Vt, lo.vd[j], st + Gm::KBYTES + (Gm::VI * w + j) * 1024);
}

// One decode iteration over the pair of tiles in stages (S0, S1): waves 0,1
// take the tile in S0, waves 2,3 the one in S1 (a 32-key slice each). Waits
// until both have landed (the other three stages stay in flight), computes
// this wave's slice, then refills S0 and S1 with the tiles five ahead.
template <int D, int S0, int S1>
__device__ __forceinline__ void narrow_iteration(
    char* smem, const LaneOffsets<D, 4>& lo4, const uint32_t (&kq)[Geo<D, 4>::KS],
    const uint32_t (&vq)[2], const u32x4 (&qop)[1][Geo<D, 4>::KS],
    f32x16 (&oacc)[1][Geo<D, 4>::DT], float (&m)[1], float (&l)[1], float c2, bool active,
    int tp, const char* Ka, const char* Va, const char* Kb, const char* Vb, int w) {
  using Gm = Geo<D, 4>;
  constexpr int SB = NarrowRing<D>::SB;
  wait_vmcnt<(kNarrowStages - 2) * Gm::PER>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read moves above the wait
  const uint32_t st = (uint32_t)(tp ? S1 * SB : S0 * SB);
  // branch-free: a wave without a tile this iteration (odd tile count) reads
  // the clamped duplicate tile and masks every score, leaving its state as is
  f32x16 sc[1];
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks)
    sc[0] = mfma_bf16(lds16(smem + st + kq[ks]), qop[0][ks], ks == 0 ? f32x16{} : sc[0]);
  if (!active) sc[0] = f32x16{} - INFINITY;
  float mx[1];
  slice_max3<1>(sc, mx);
  rescale_top<1, Gm::DT>(mx, m, l, oacc, c2);
  u32x4 p[1][2];
  slice_exp2<1>(sc, m, l, p, c2);
#pragma unroll
  for (int dt = 0; dt < Gm::DT; ++dt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      oacc[0][dt] = mfma_bf16(lds16(smem + st + vq[kb] + dt * 32 * 128), p[0][kb], oacc[0][dt]);
  block_sync_lds();
  dma_stage_narrow<D, S0>(smem, Ka, Va, lo4, w);
  dma_stage_narrow<D, S1>(smem, Kb, Vb, lo4, w);
}

// Decode partial kernel. One workgroup per (sequence, kv head, range or
// split); its interior 64-key tiles stream through a ring of five LDS stages
// by direct-to-LDS loads, two tiles per iteration with the next three in
// flight. Waves 0,1 take the 32-key slices of the even tile, waves 2,3 those
// of the odd tile, each with its own softmax state; the four states are
// merged through LDS at the end. Sized so one workgroup per CU streams a
// long contiguous key range with 96-160 KB of loads outstanding.
template <int D, bool FUSED, bool PAGED>
__global__ __launch_bounds__(256) void attn_narrow_kernel(const NarrowArgs a) {
  using Gm = Geo<D, 4>;
  using Ring = NarrowRing<D>;
  constexpr int KS = Gm::KS, DT = Gm::DT;
  // after the stream the ring holds the merge area: per wave, O as [D][33]
  // (padded: conflict-free both ways), then m and l
  constexpr int OSM_BYTES = 4 * D * 33 * 4;
  static_assert(OSM_BYTES + 2 * 4 * 32 * 4 <= Ring::BYTES, "merge area must fit in the ring");
  static_assert(Gm::V_AT + Gm::VBYTES <= Ring::BYTES, "edge tiles must fit in the ring");
  static_assert(32 * D * 2 <= Ring::SB, "query tile must fit in one stage");
  __shared__ __attribute__((aligned(1024))) char smem[Ring::BYTES];
  // the wave index is uniform: keep it (and what derives from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int tp = w >> 1, kt = w & 1;  // tile of the pair, 32-key slice of the tile

  // splits in reverse order: the short, partly masked tail splits start
  // first instead of waiting for a CU after the long context splits
  int32_t gidx, sigma;
  narrow_map(blockIdx.x, a.NG, a.n_split, &gidx, &sigma);
  const int kvh = gidx % a.Hkv, s = gidx / a.Hkv;
  int64_t lo, hi;
  int32_t host;
  split_rows(a.L, a.blk, a.n_blocks, a.per_block, a.blk_len, a.tail_len, a.kv_len, sigma, &lo, &hi,
             &host);
  const int64_t pos0 = a.kv_len - a.n_query;
  const int ncols = (int)(a.n_query * a.G);
  // column l32 -> (query j, head)
  const int cj = l32 / a.G, ch = kvh * a.G + l32 % a.G;
  const bool cvalid = l32 < ncols;
  const int64_t cpos = pos0 + cj;

  const int64_t head_row0 = ((int64_t)s * a.Hkv + kvh) * a.rows;
  const uint16_t* K = PAGED ? a.k : a.k + head_row0 * D;
  const uint16_t* V = PAGED ? a.v : a.v + head_row0 * D;
  // element offset of this (sequence, kv head)'s tile t from K and from V
  auto tile_at = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem<true, D>(a.pm, a.rows, a.Hkv, s, kvh, t);
    else return t * 64 * D;
  };
  // the same for a wave-uniform t (a scalar table read)
  auto tile_at_u = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem_u<true, D>(a.pm, a.rows, a.Hkv, s, kvh, t);
    else return t * 64 * D;
  };
  const float c2 = a.c2;

  if (FUSED) {
    // append: this split's share of the new rows [pos0, kv_len) goes into the
    // cache before any of its tiles is loaded (no other split reads them)
    const int64_t r0 = pos0 > lo ? pos0 : lo;
    const int64_t r1 = a.kv_len < hi ? a.kv_len : hi;
    if (r1 > r0) {
      uint16_t* Kw = (uint16_t*)K;
      uint16_t* Vw = (uint16_t*)V;
      const int n = (int)(r1 - r0);
      for (int u = tid; u < n * D; u += 256) {
        const int rr = u / D, e = u % D;
        const int64_t r = r0 + rr;
        const int64_t src = (((int64_t)s * a.n_query + (r - pos0)) * a.Hkv + kvh) * D + e;
        const int64_t tb = tile_at(r / 64);
        Kw[tb + (r % 64) * D + e] = a.k_new[src];
        Vw[tb + e * 64 + (r % 64)] = a.v_new[src];
      }
      // the stores must complete before this workgroup loads those rows;
      // every other split never reads them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
    }
  }

  f32x16 oacc[1][DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[0][dt] = f32x16{};
  float m[1] = {kMinit}, l[1] = {0.0f};

  u32x4 qop[1][KS];
  auto load_q = [&](u32x4 (&q)[1][KS]) {
    const uint16_t* qp = a.q + (((int64_t)s * a.n_query + (cvalid ? cj : 0)) * a.Hq + ch) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[0][ks] = cvalid ? ld16(qp + (2 * ks + g) * 8) : u32x4{0, 0, 0, 0};
  };

  // interior tiles: inside [lo, hi) and not after any query position
  const TileRuns runs = tile_runs(0, lo, hi, pos0);
  const int64_t bf = runs.bf, bl = runs.bl, i0 = runs.i0, i1 = runs.i1;
  const int n_int = (int)(i1 - i0);

  if (n_int > 0) {
    LaneOffsets<D, 4> lo4;
    lo4.init(l32, g, w, lane);
    // this wave's operand offsets inside a stage: its 32-key slice
    uint32_t kq[KS], vq[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kq[ks] = lo4.kq[ks] + kt * 32 * Gm::RB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      vq[kb] = (uint32_t)Gm::KBYTES + v_off(l32, 4 * kt + 2 * kb + g);
    const char* Kc = (const char*)K;
    const char* Vc = (const char*)V;
    const int jmax = n_int - 1;
#define STAR_TOFF(j) (tile_at_u(i0 + ((j) < jmax ? (j) : jmax)) * 2)
    const int n_it = (n_int + 1) / 2;
    // the query tile arrives by the same direct-to-LDS loads, into stage 4
    // before that stage's first tile: 16-byte chunk u (lane-major over the
    // wave's QI loads) of column u / CH, d-chunk u % CH, lands at byte 16 u.
    // A column past ncols loads column 0 and is zeroed when read.
    constexpr int QI = 32 * D * 2 / 1024 / 4;  // 1-KB loads per wave
    char* qsm = smem + 4 * Ring::SB;
    const char* qbase = (const char*)(a.q + (int64_t)s * a.n_query * a.Hq * D);
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int u = (w * QI + i) * 64 + lane;
      const int c = u / Gm::CH, k = u % Gm::CH;
      const int cc = c < ncols ? c : 0;
      const uint32_t off =
          (uint32_t)((((cc / a.G) * a.Hq + kvh * a.G + cc % a.G) * D + k * 8) * 2);
      dma16_lds(qbase, off, qsm + (w * QI + i) * 1024);
    }
    dma_stage_narrow<D, 0>(smem, Kc + STAR_TOFF(0), Vc + STAR_TOFF(0), lo4, w);
    dma_stage_narrow<D, 1>(smem, Kc + STAR_TOFF(1), Vc + STAR_TOFF(1), lo4, w);
    dma_stage_narrow<D, 2>(smem, Kc + STAR_TOFF(2), Vc + STAR_TOFF(2), lo4, w);
    dma_stage_narrow<D, 3>(smem, Kc + STAR_TOFF(3), Vc + STAR_TOFF(3), lo4, w);
    // the query loads are the oldest: wait for them alone, then every wave
    // reads its B operand from LDS (no register load the compiler would
    // drain), and stage 4 gets its tile once every wave has read it
    wait_vmcnt<4 * Gm::PER>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = lds16(qsm + l32 * (D * 2) + (2 * ks + g) * 16);
      qop[0][ks] = cvalid ? v : u32x4{0, 0, 0, 0};
    }
    block_sync_lds();
    dma_stage_narrow<D, 4>(smem, Kc + STAR_TOFF(4), Vc + STAR_TOFF(4), lo4, w);
    // iteration k takes tiles 2k, 2k + 1 from stages (2k) % 5, (2k + 1) % 5
#define STAR_ITER(S0, S1, K)                                                                  \
  {                                                                                           \
    const int t0 = 2 * (K);                                                                   \
    narrow_iteration<D, S0, S1>(smem, lo4, kq, vq, qop, oacc, m, l, c2, t0 + tp < n_int, tp,  \
                                Kc + STAR_TOFF(t0 + 5), Vc + STAR_TOFF(t0 + 5),               \
                                Kc + STAR_TOFF(t0 + 6), Vc + STAR_TOFF(t0 + 6), w);           \
  }
    for (int k = 0; k < n_it; k += 5) {
      STAR_ITER(0, 1, k)
      if (k + 1 >= n_it) break;
      STAR_ITER(2, 3, k + 1)
      if (k + 2 >= n_it) break;
      STAR_ITER(4, 0, k + 2)
      if (k + 3 >= n_it) break;
      STAR_ITER(1, 2, k + 3)
      if (k + 4 >= n_it) break;
      STAR_ITER(3, 4, k + 4)
    }
#undef STAR_ITER
#undef STAR_TOFF
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }

  if (n_int == 0) load_q(qop);

  // edge tiles (the causal tail, unaligned ends): waves 0,1, masked
  const int n_edge = (int)(i0 - bf) + (int)(bl - i1);
  if (n_edge > 0) {
    for (int e = 0; e < n_edge; ++e) {
      const int64_t kbase = (e < i0 - bf ? bf + e : i1 + (e - (i0 - bf))) * 64;
      EdgeTile<D, 4> et;
      et.load(K + tile_at_u(kbase / 64), V + tile_at_u(kbase / 64), kbase, lo, hi, tid);
      et.store(smem, tid);
      block_sync_lds();
      if (tp == 0) {
        f32x16 sc[1];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[0] = mfma_bf16(lds16(smem + k_off<D>(l32, 2 * ks + g) + kt * 32 * Gm::RB),
                            qop[0][ks], ks == 0 ? f32x16{} : sc[0]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = kbase + 32 * kt + acc_key(i, g);
          if (key < lo || key >= hi || key > cpos || !cvalid) sc[0][i] = -INFINITY;
        }
        float mx[1];
        slice_max3<1>(sc, mx);
        rescale_top<1, DT>(mx, m, l, oacc, c2);
        u32x4 p[1][2];
        slice_exp2<1>(sc, m, l, p, c2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            oacc[0][dt] = mfma_bf16(
                lds16(smem + Gm::V_AT + v_off(l32, 4 * kt + 2 * kb + g) + dt * 32 * 128), p[0][kb],
                oacc[0][dt]);
      }
      block_sync_lds();
    }
  }

  // ---- merge the four waves' (m, l, O) and write the split's partial (the
  // ring is idle here: every load has landed and every read is done)
  float* osm = (float*)smem;                   // [4][D][33]: padded, no bank conflicts
  float* msm = (float*)(smem + OSM_BYTES);     // [4][32]
  float* lsm = msm + 4 * 32;                   // [4][32]
  {
    const float lw = pair_sum(l[0]);
    if (g == 0) {
      msm[w * 32 + l32] = m[0];
      lsm[w * 32 + l32] = lw;
    }
    if (cvalid) {
      float* ow = osm + w * D * 33 + l32;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ow[(32 * dt + 8 * (i >> 2) + 4 * g + (i & 3)) * 33] = oacc[0][dt][i];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < ncols * D; idx += 256) {
    const int c = idx / D, e = idx - c * D;
    float M = msm[c];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, msm[ww * 32 + c]);
    float Ls = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = fast_exp2((msm[ww * 32 + c] - M) * c2);
      Ls += f * lsm[ww * 32 + c];
      O += f * osm[(ww * D + e) * 33 + c];
    }
    const int j = c / a.G, h = kvh * a.G + c % a.G;
    const int64_t base = (((int64_t)s * a.n_query + j) * a.Hq + h) * a.n_split + sigma;
    const bool any = Ls > 0.0f;
    a.o_part[base * D + e] = any ? O / Ls : 0.0f;
    if (e == 0) a.lse_part[base] = any ? M * a.scale + logf(Ls) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for the balanced plan: every wave streams one range of the
// plan (a contiguous run of cache rows of one sequence and kv head) through a
// ring of its own, two stages of one 32-key slice each ([K rows | V^T
// columns]), with its own copy of the query tile. No wave waits for another:
// there is no barrier in the kernel. Each wave writes the partial of its
// range (two, if the range holds a host boundary) straight from registers.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;      // [B][n_query][Hq][D]
  float* o_part;
  float* lse_part;
  const uint16_t* k_new;  // FUSED: [B][n_query][Hkv][D], written at kv_len - n_query
  const uint16_t* v_new;
  int64_t rows, L, blk, kv_len, n_query, wg_rows, bnd_period;
  int32_t n_split, n_blocks, n_wg;  // n_wg: ranges per (sequence, kv head)
  int32_t Hq, Hkv, G, NG, WPG;      // WPG: workgroups per (sequence, kv head)
  float scale, c2;
  PageMap pm;                       // paged cache
};

template <int D>
struct DecodeGeo {
  static constexpr int CH = D / 8;        // 16-byte chunks per K row
  static constexpr int RB = 2 * D;        // bytes per K row
  static constexpr int KB = 32 * RB;      // K rows of a slice
  static constexpr int VB = D * 64;       // V^T of a slice: D rows x 32 keys
  static constexpr int SB = KB + VB;      // one stage
  static constexpr int QB = 32 * D * 2;   // query tile, 32 columns
  static constexpr int WB = 2 * SB + QB;  // one wave's LDS
  static constexpr int KI = KB / 1024, VI = VB / 1024, QI = QB / 1024;  // 1-KB loads
  static constexpr int PER = KI + VI;     // loads per slice
  static constexpr int KS = D / 16, DT = D / 32;
};

// LDS byte offset of 16-byte chunk kc (keys 8 kc .. 8 kc + 7 of the slice) of
// row e of a V^T slice. The XOR with bits 2..3 of e spreads the 16 lanes of
// one LDS cycle (rows e .. e + 15, one kc) over all banks.
__device__ __forceinline__ uint32_t vs_off(int e, int kc) {
  return (uint32_t)(e * 64 + ((kc ^ ((e >> 2) & 3)) << 4));
}

// MID: a host boundary may fall inside a 32-key slice (a context or block
// length off the slice grid); only then is the slice-splitting path compiled.
template <int D, bool FUSED, bool PAGED, bool MID>
__global__ __launch_bounds__(256) void attn_decode_kernel(const DecodeArgs a) {
  using Dg = DecodeGeo<D>;
  constexpr int KS = Dg::KS, DT = Dg::DT;
  __shared__ __attribute__((aligned(1024))) char smem[4 * Dg::WB];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  char* ring = smem + w * Dg::WB;   // this wave's two stages
  char* qsm = ring + 2 * Dg::SB;    // and its query tile

  // the workgroup holding the last ranges (the tail, the appended rows) first
  int32_t gidx;
  int64_t r;
  decode_map(blockIdx.x, w, a.NG, a.WPG, &gidx, &r);
  if (r >= a.n_wg) return;
  const int kvh = gidx % a.Hkv, s = gidx / a.Hkv;
  const int64_t pos0 = a.kv_len - a.n_query;
  // split sigma from lo; with a host boundary bnd inside, split sigma + 1 from bnd
  const DecodeRange rg =
      decode_range(r, a.wg_rows, a.kv_len, a.L, a.blk, a.n_blocks, a.bnd_period, pos0);
  const int64_t lo = rg.lo, hi = rg.hi, bnd = rg.bnd;
  const int32_t sigma = rg.sigma;
  const int ncols = (int)(a.n_query * a.G);
  const int cj = l32 / a.G, ch = kvh * a.G + l32 % a.G;  // column l32 -> (query, head)
  const bool cvalid = l32 < ncols;
  const int64_t cpos = pos0 + cj;
  const int64_t head_row0 = ((int64_t)s * a.Hkv + kvh) * a.rows;
  const uint16_t* K = PAGED ? a.k : a.k + head_row0 * D;
  const uint16_t* V = PAGED ? a.v : a.v + head_row0 * D;
  // element offset of this (sequence, kv head)'s tile t from K and from V
  auto tile_at = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem<true, D>(a.pm, a.rows, a.Hkv, s, kvh, t);
    else return t * 64 * D;
  };
  // the same for a wave-uniform t (a scalar table read)
  auto tile_at_u = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem_u<true, D>(a.pm, a.rows, a.Hkv, s, kvh, t);
    else return t * 64 * D;
  };
  const float c2 = a.c2;

  if (FUSED) {
    // append this range's share of the new rows before any of its slices is
    // loaded (no other wave reads them); the stores complete before the loads
    const int64_t r0 = pos0 > lo ? pos0 : lo;
    const int64_t r1 = a.kv_len < hi ? a.kv_len : hi;
    if (r1 > r0) {
      uint16_t* Kw = (uint16_t*)K;
      uint16_t* Vw = (uint16_t*)V;
      const int n = (int)(r1 - r0);
      for (int u = lane; u < n * D; u += 64) {
        const int rr = u / D, e = u % D;
        const int64_t row = r0 + rr;
        const int64_t src = (((int64_t)s * a.n_query + (row - pos0)) * a.Hkv + kvh) * D + e;
        const int64_t tb = tile_at(row / 64);
        Kw[tb + (row % 64) * D + e] = a.k_new[src];
        Vw[tb + e * 64 + (row % 64)] = a.v_new[src];
      }
      wait_vmcnt<0>();
    }
  }

  // ---- this wave's load offsets (bytes) inside a slice
  uint32_t kd[Dg::KI], vd[Dg::VI];
#pragma unroll
  for (int j = 0; j < Dg::KI; ++j) {
    // LDS slot (j * 1024 + 16 lane) / RB of the K slice holds key row swap23(slot)
    const int slot = j * (1024 / Dg::RB) + lane / Dg::CH;
    const int c = (lane % Dg::CH) ^ (slot & (Dg::CH - 1));
    kd[j] = (uint32_t)(swap23(slot) * Dg::RB + 16 * c);
  }
#pragma unroll
  for (int j = 0; j < Dg::VI; ++j) {
    const int e = 16 * j + lane / 4;
    const int kc = (lane & 3) ^ ((e >> 2) & 3);
    vd[j] = (uint32_t)(e * 128 + 16 * kc);  // inside the V^T tile of the slice's 64 rows
  }
  // operand offsets: K rows (slot l32, chunk 2 ks + g), V^T rows (32 dt + l32, chunk 2 kb + g)
  uint32_t kq[KS], vq[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kq[ks] = k_off<D>(l32, 2 * ks + g);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) vq[kb] = (uint32_t)Dg::KB + vs_off(l32, 2 * kb + g);

  // slices of [lo, hi): [0, n_in) fully visible to every column and inside
  // [lo, hi); [n_in, n_sl) masked (range end not on a slice, or keys after
  // the first query position)
  const int n_sl = rg.n_sl;
  const int n_in = rg.n_in;
  // split 2 starts in slice sb; if bnd is not on a slice edge, that slice's
  // keys below bnd still belong to split 1
  const int sb = bnd >= 0 ? (int)((bnd - lo) / 32) : 0x7fffffff;
  const bool bnd_mid = MID && bnd >= 0 && (bnd - lo) % 32 != 0;
  const char* Kc = (const char*)K;
  const char* Vc = (const char*)V;
  // slice i (clamped to the last one): K rows from row lo + 32 i; V^T from the
  // 64-row tile holding them, half (lo / 32 + i) & 1
  auto k_at = [&](int i) -> const char* {
    i = i < n_sl ? i : n_sl - 1;
    const int64_t row = lo + 32 * (int64_t)i;
    return Kc + tile_at_u(row / 64) * 2 + (row % 64) * Dg::RB;
  };
  auto v_at = [&](int i) -> const char* {
    i = i < n_sl ? i : n_sl - 1;
    const int64_t row = lo + 32 * (int64_t)i;
    return Vc + tile_at_u(row / 64) * 2 + (row % 64) * 2;
  };
  auto load_slice_at = [&](int st, const char* kt, const char* vt) {
    char* d = ring + st * Dg::SB;
    // K rows of a slice are whole 128-byte lines: non-temporal. The slice's
    // V^T is half of each line of its tile (32 of 64 keys); the next slice
    // reads the other half from L2, which a non-temporal load would not leave
    // there (measured: 20% slower per step, against 15% faster for K alone)
#pragma unroll
    for (int j = 0; j < Dg::KI; ++j) dma16_lds<true>(kt, kd[j], d + j * 1024);
#pragma unroll
    for (int j = 0; j < Dg::VI; ++j) dma16_lds<false>(vt, vd[j], d + Dg::KB + j * 1024);
  };
  auto load_slice = [&](int st, int i) { load_slice_at(st, k_at(i), v_at(i)); };

  // ---- query tile: chunk u of this wave's QI loads = column u / CH, chunk
  // (u % CH) ^ (column & (CH - 1)) at LDS k_off(column, chunk); a column past
  // ncols loads column 0 and is zeroed when read
  {
    const char* qbase = (const char*)(a.q + (int64_t)s * a.n_query * a.Hq * D);
#pragma unroll
    for (int i = 0; i < Dg::QI; ++i) {
      const int col = i * (1024 / Dg::RB) + lane / Dg::CH;
      const int c = (lane % Dg::CH) ^ (col & (Dg::CH - 1));
      const int cc = col < ncols ? col : 0;
      const uint32_t off =
          (uint32_t)((((cc / a.G) * a.Hq + kvh * a.G + cc % a.G) * D + c * 8) * 2);
      dma16_lds(qbase, off, qsm + i * 1024);
    }
  }
  // loads are issued for slices inside the range only; every wait below
  // counts exactly the slices still in flight
  load_slice(0, 0);
  if (n_sl > 1) {
    load_slice(1, 1);
    wait_vmcnt<2 * Dg::PER>();  // the query tile (the oldest loads) has landed
  } else {
    wait_vmcnt<Dg::PER>();
  }
  asm volatile("" ::: "memory");
  u32x4 qop[1][KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 v = lds16(qsm + kq[ks]);
    qop[0][ks] = cvalid ? v : u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[1][DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[0][dt] = f32x16{};
  float m[1] = {kMinit}, l[1] = {0.0f};
  f32x16 oprev[1][DT];
  float mprev = kMinit, lprev = 0.0f;
  bool switched = false;

  // paged cache: the page id of the next refill's tile (slice i + 2 in step
  // i), read right after the previous refill, so that the scalar load lands
  // while the step waits for its slice; the address is formed at the refill
  auto slice_page = [&](int i) -> int32_t {
    i = i < n_sl ? i : n_sl - 1;
    return page_u(a.pm, s, (lo + 32 * (int64_t)i) / 64);
  };
  int32_t npg = 0;
  if constexpr (PAGED) npg = slice_page(2);
  // close split 1 (its state moves to oprev) and open split 2
  auto switch_split = [&]() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      oprev[0][dt] = oacc[0][dt];
      oacc[0][dt] = f32x16{};
    }
    mprev = m[0];
    lprev = l[0];
    m[0] = kMinit;
    l[0] = 0.0f;
    switched = true;
  };
  auto step = [&](int i, int st) {
    // slice i has landed; slice i + 1 (if any) stays in flight
    if (i + 1 < n_sl) wait_vmcnt<Dg::PER>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    const bool split_here = bnd_mid && i == sb;
    if (i >= sb && !switched && !split_here) switch_split();
    char* sm = ring + st * Dg::SB;
    const bool masked = i >= n_in;
    const int64_t key0 = lo + 32 * (int64_t)i;
    if (masked) {
      // keys at or past hi are rows nobody wrote: zero their V^T elements
      for (int u = lane; u < D * 4; u += 64) {
        const int e = u / 4, kc = u % 4;
        u32x4* pc = (u32x4*)(sm + Dg::KB + vs_off(e, kc));
        *pc = mask_chunk(*pc, key0 + 8 * kc, lo, hi);
      }
    }
    f32x16 sc[1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sc[0] = mfma_bf16(lds16(sm + kq[ks]), qop[0][ks], ks == 0 ? f32x16{} : sc[0]);
    if (masked) {
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int64_t key = key0 + acc_key(ii, g);
        if (key >= hi || key > cpos || !cvalid) sc[0][ii] = -INFINITY;
      }
    }
    // online-softmax update of the current split with scores t
    auto update = [&](f32x16 (&t)[1]) {
      float mx[1];
      slice_max3<1>(t, mx);
      rescale_top<1, DT>(mx, m, l, oacc, c2);
      u32x4 p[1][2];
      slice_exp2<1>(t, m, l, p, c2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          oacc[0][dt] = mfma_bf16(lds16(sm + vq[kb] + dt * 32 * 64), p[0][kb], oacc[0][dt]);
    };
    if (split_here) {
      // the host boundary falls inside this slice: its keys below bnd end
      // split 1, the rest start split 2 (both are written rows)
      f32x16 s1[1] = {sc[0]};
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        if (key0 + acc_key(ii, g) >= bnd) s1[0][ii] = -INFINITY;
        else sc[0][ii] = -INFINITY;
      }
      update(s1);
      switch_split();
    }
    update(sc);
    // this wave's reads of the stage are complete before it is refilled
    if (i + 2 < n_sl) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      if constexpr (PAGED) {
        const int64_t row = lo + 32 * (int64_t)(i + 2);
        const int64_t tb = ((int64_t)npg * a.Hkv + kvh) * (64 * D) * 2;
        load_slice_at(st, Kc + tb + (row % 64) * Dg::RB, Vc + tb + (row % 64) * 2);
        npg = slice_page(i + 3);
      } else {
        load_slice(st, i + 2);
      }
    }
  };
  for (int i = 0; i < n_sl; i += 2) {
    step(i, 0);
    if (i + 1 >= n_sl) break;
    step(i + 1, 1);
  }
  wait_vmcnt<0>();
  // a split that starts at bnd after the last slice is empty
  if (bnd >= 0 && !switched) switch_split();

  // ---- partials straight from registers: column l32's 16 values per dt
  // tile are rows 32 dt + 8 (i / 4) + 4 g + (i % 4)
  auto write_split = [&](int32_t sg, const f32x16 (&oa)[1][DT], float mw, float lraw) {
    const float lt = pair_sum(lraw);
    if (!cvalid) return;
    const bool any = lt > 0.0f;
    const float inv = any ? 1.0f / lt : 0.0f;
    const int64_t base = (((int64_t)s * a.n_query + cj) * a.Hq + ch) * a.n_split + sg;
    float* op = a.o_part + base * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4*)(op + 32 * dt + 8 * i4 + 4 * g) =
            float4{oa[0][dt][4 * i4] * inv, oa[0][dt][4 * i4 + 1] * inv,
                   oa[0][dt][4 * i4 + 2] * inv, oa[0][dt][4 * i4 + 3] * inv};
    if (g == 0) a.lse_part[base] = any ? mw * a.scale + logf(lt) : -INFINITY;
  };
  if (bnd >= 0) {
    write_split(sigma, oprev, mprev, lprev);
    write_split(sigma + 1, oacc, m[0], l[0]);
  } else {
    write_split(sigma, oacc, m[0], l[0]);
  }
}

// fp32 path arguments (phase 1 and the phase-2 partials)
struct F32Args {
  const float* k;
  const float* v;
  const float* q;
  float* o;
  float* o_part;
  float* lse_part;
  int64_t rows, q_tokens, L, blk, anc, kv_len;
  int64_t blk_len, tail_len;
  int32_t per_block, n_split, n_blocks;
  int32_t Hq, Hkv, G;
  float scale;
  PageMap pm;  // phase 2 on a paged cache
  const float* rope_cos;  // ROPE (phase 1): tables [n_pos][D/2]
  const float* rope_sin;
};

// ---------------------------------------------------------------------------
// fp32 on the matrix cores (phase 1, with or without a rotary embedding, and
// the phase-2 partials): one workgroup per 32 columns, v_mfma_f32_32x32x2_f32
// for both products; the workgroup's 32-key slices are dealt round robin to
// its waves, whose states merge at the end. Per slice the K rows and the V
// rows (turned back from the transposed tile) are staged in the wave's LDS
// buffers, rows outside the workgroup's key range zero;
// S^T = K Q^T (A: K[key][2 ks + g], B: Q[column][2 ks + g]); each lane then
// holds column l32 and keys 8 (r / 4) + 4 g + r % 4 of the slice; the online
// softmax runs per column in fp32 (the lane pair l32, l32 + 32 shares a
// column); P goes through LDS into the B layout of O^T += V^T P^T.
// Phase 1: columns are 32 context rows of one head, each seeing the anchor
// (blocks >= 1) and its own block causally. Phase 2: columns are (query row,
// head) pairs of one kv head, each seeing split sigma's rows up to its own
// position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int acc_row(int r, int g) { return ((r >> 2) << 3) + (g << 2) + (r & 3); }

// Bit j set for the keys k0 + j (j < 32) that lie in [lo, hi).
__device__ __forceinline__ uint32_t range_bits(int64_t lo, int64_t hi, int64_t k0) {
  const int64_t a = lo - k0 < 0 ? 0 : (lo - k0 > 32 ? 32 : lo - k0);
  const int64_t b = hi - k0 < 0 ? 0 : (hi - k0 > 32 ? 32 : hi - k0);
  const uint32_t below_b = b >= 32 ? 0xFFFFFFFFu : (1u << b) - 1u;
  const uint32_t below_a = a >= 32 ? 0xFFFFFFFFu : (1u << a) - 1u;
  return b > a ? below_b & ~below_a : 0u;
}

template <int D, bool PHASE1, bool PAGED, int ROPE>
__global__ __launch_bounds__(64 * f32m_waves(D)) void attn_f32m_kernel(const F32Args a) {
  static_assert(!(PHASE1 && PAGED), "phase 1 reads the contiguous cache");
  static_assert(PHASE1 || ROPE == kRopeNone, "rotary embedding is fused into phase 1");
  constexpr int DT = D / 32;  // O^T tiles of 32 dimensions
  constexpr int LD = D + 1;   // padded LDS rows
  constexpr bool ADJ = ROPE == kRopeAdjacent;
  constexpr int NW = f32m_waves(D);  // waves; slice i of the workgroup goes to wave i % NW
  __shared__ float sQ[32 * LD];
  __shared__ float sQa[ADJ ? 32 * LD : 1];  // adjacent ids: the query turned back for the anchor
  __shared__ float sKw[NW * 32 * LD];       // per wave: K rows, V^T rows, P
  __shared__ float sVw[NW * 32 * LD];
  __shared__ float sPw[NW * 32 * 33];
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5, w = threadIdx.x >> 6;
  float* const sK = sKw + w * 32 * LD;
  float* const sV = sVw + w * 32 * LD;
  float* const sP = sPw + w * 32 * 33;
  const int64_t wid = blockIdx.x;

  // the workgroup's columns: column c -> (token row in q, head), valid, and its
  // visible keys: [0, hiA) (phase 1) and [loB, hiB) up to its position
  int64_t s, ncg = 0, rg = 0, cg = 0;
  int32_t h0 = 0, kvh, sigma = 0;
  int64_t lo = 0, hi = 0;  // phase 2: the split's rows
  if (PHASE1) {
    f32m_phase1_map(wid, a.L, a.Hq, &s, &h0, &rg);
    kvh = h0 / a.G;
  } else {
    ncg = cdiv_hd(a.q_tokens * a.G, 32);
    f32m_phase2_map(wid, a.n_split, ncg, a.Hkv, &s, &kvh, &cg, &sigma);
    int32_t host;
    split_rows(a.L, a.blk, a.n_blocks, a.per_block, a.blk_len, a.tail_len, a.kv_len, sigma, &lo,
               &hi, &host);
  }
  auto col = [&](int c) {
    return f32m_column(PHASE1, c, PHASE1 ? rg : cg, PHASE1 ? h0 : kvh, a.L, a.blk, a.anc,
                       a.q_tokens, a.G, a.kv_len, lo, hi);
  };
  // the workgroup's key range: the union of its columns' ranges (uniform)
  int64_t kA, kB0, kB1;
  f32m_wave_keys(PHASE1, PHASE1 ? rg : cg, PHASE1 ? h0 : kvh, a.L, a.blk, a.anc, a.q_tokens, a.G,
                 a.kv_len, lo, hi, &kA, &kB0, &kB1);
  const int64_t head_row0 = (s * a.Hkv + kvh) * a.rows;
  const float* K = PAGED ? a.k : a.k + head_row0 * D;
  const float* V = PAGED ? a.v : a.v + head_row0 * D;
  auto tile_at = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) return tile_elem<true, D>(a.pm, a.rows, a.Hkv, (int)s, (int)kvh, t);
    else return t * 64 * D;
  };
  // the keys of slice [k0, k0 + 32) that are loaded (else zero): those some
  // column of the workgroup may see, as a bit mask
  auto slice_bits = [&](int64_t k0) { return range_bits(0, kA, k0) | range_bits(kB0, kB1, k0); };
  // x, or +0 where bit j of m is clear, on the bits: the pieces hold the
  // unwritten (possibly NaN) rows next to wanted keys, and a floating-point
  // select of a NaN is not something the no-NaN build may keep
  auto keep = [](float x, uint32_t m, int j) {
    return __uint_as_float(__float_as_uint(x) & (0u - ((m >> j) & 1u)));
  };

  // the columns' queries; with a rotary embedding turned at the column's
  // position id (pairs e, e + D/2), and for adjacent anchor ids also turned
  // back by i*b - a for the anchor's keys (rotations compose: the cached
  // anchor keys stay at their own row ids)
  // Each lane works out its own column once (the map divides by the block
  // length); an iteration's column c is the same on every lane, so its fields
  // come from lane c by readlane.
  const F32mCol me = col(l32);
  auto from_lane = [](int64_t v, int c) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, c);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), c);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  for (int k = w; k < 32 * D / 64; k += NW) {  // the waves share the staging
    const int c = 64 * k / D, e = (lane + 64 * k) % D;  // element u = lane + 64 k: column u / D
    F32mCol x;
    x.valid = __builtin_amdgcn_readlane((int)me.valid, c) != 0;
    x.row = from_lane(me.row, c);
    x.head = __builtin_amdgcn_readlane(me.head, c);
    x.hiA = from_lane(me.hiA, c);
    float vb = 0.0f, va = 0.0f;
    if (x.valid) {
      const float* qp = a.q + ((s * a.q_tokens + x.row) * a.Hq + x.head) * D;
      if constexpr (ROPE == kRopeNone) {
        vb = qp[e];
      } else {
        const int e2 = e < D / 2 ? e : e - D / 2;
        const float qx = qp[e2], qy = qp[e2 + D / 2];
        auto turn = [&](int64_t id) {
          const float cc = a.rope_cos[id * (D / 2) + e2], sn = a.rope_sin[id * (D / 2) + e2];
          return e < D / 2 ? rope_a(qx, qy, cc, sn) : rope_b(qx, qy, cc, sn);
        };
        vb = turn(x.row);
        if constexpr (ADJ) va = turn(x.hiA > 0 ? x.row - ((x.row / a.blk) * a.blk - a.anc) : x.row);
      }
    }
    sQ[c * LD + e] = vb;
    if constexpr (ADJ) sQa[c * LD + e] = va;
  }
  __syncthreads();
  // d = 64: the B operands of S^T = K Q^T stay in registers for the whole
  // loop; d = 128 reads them from LDS with the K operands (registers would
  // spill next to the slice prefetch)
  constexpr bool QREG = D <= 64;
  float qop[QREG ? D / 2 : 1], qaop[QREG && ADJ ? D / 2 : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) {
      qop[ks] = sQ[l32 * LD + 2 * ks + g];
      if constexpr (ADJ) qaop[ks] = sQa[l32 * LD + 2 * ks + g];
    }
  }
  // 16 k-steps of S^T from K and the query copy qs (registers qr or LDS)
  auto qk16 = [&](f32x16 acc, int k16, const float* qr, const float* qs) {
    float kop[16], qch[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kop[j] = sK[l32 * LD + 2 * (16 * k16 + j) + g];
      qch[j] = QREG ? qr[16 * k16 + j] : qs[l32 * LD + 2 * (16 * k16 + j) + g];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kop[j], qch[j], acc, 0, 0, 0);
    return acc;
  };
  float m = kMinit, l = 0.0f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

  // A slice's K and V go through registers in 16-byte pieces: all of a
  // slice's loads are issued one slice ahead, so they land during the
  // arithmetic of the slice before. Piece f = lane + 64 i of K is key f/(D/4),
  // dimensions 4 (f % (D/4)) + 0..3; piece f of V^T is dimension f / 8, keys
  // 4 (f % 8) + 0..3. A piece whose keys no column sees reads row 0 (always
  // written); every element of a key no column sees is stored as zero.
  constexpr int NF = D / 8;  // pieces of each matrix per lane
  f32x4 kr[NF], vr[NF];
  // a slice lies inside one 64-key tile: its K rows and V^T columns start at
  // one base each; a piece no column wants reads tile 0 (row 0 is written)
  const float* const K0 = K + tile_at(0);
  const float* const V0 = V + tile_at(0);
  auto fetch = [&](int64_t k0) {
    const uint32_t wm = slice_bits(k0);
    const int64_t t = tile_at(k0 / 64);
    const float* const Kb = K + t + (k0 % 64) * D;
    const float* const Vb = V + t + (k0 % 64);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int f = lane + 64 * i;
      const int j = f / (D / 4), e = 4 * (f % (D / 4));
      kr[i] = *(const f32x4*)(((wm >> j) & 1u) ? Kb + j * D + e : K0 + e);
      const int dv = f / 8, kq = 4 * (f % 8);
      vr[i] = *(const f32x4*)(((wm >> kq) & 15u) ? Vb + dv * 64 + kq : V0 + dv * 64);
    }
  };
  // the workgroup's slices (those some column sees), dealt round robin to
  // the waves; every wave meets every barrier of the rounds
  const F32mSlices sl = f32m_slices(kA, kB0, kB1);
  const int64_t rounds = cdiv_hd(sl.n, NW);
  if (w < sl.n) fetch(f32m_slice_at(sl, w));
  for (int64_t rd = 0, si = w; rd < rounds; ++rd, si += NW) {
    const bool act = si < sl.n;
    const int64_t k0 = act ? f32m_slice_at(sl, si) : 0;
    __syncthreads();  // the previous slice's LDS reads are done
    if (act) {
      const uint32_t wm = slice_bits(k0);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int f = lane + 64 * i;
        const int kk = f / (D / 4), e = 4 * (f % (D / 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) sK[kk * LD + e + c] = keep(kr[i][c], wm, kk);
        const int ev = f / 8, kv = 4 * (f % 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) sV[(kv + c) * LD + ev] = keep(vr[i][c], wm, kv + c);
      }
    }
    __syncthreads();
    if (si + NW < sl.n) fetch(f32m_slice_at(sl, si + NW));
    if (act) {  // (a wave with no slice this round only meets the barriers)
      // the operands are read 16 k-steps ahead of their MFMAs
      f32x16 sc = f32x16{};
#pragma unroll
      for (int k16 = 0; k16 < D / 32; ++k16) sc = qk16(sc, k16, qop, sQ);
      if constexpr (ADJ) {
        if (k0 < kA) {  // anchor keys of blocks >= 1: scores with the turned-back query
          f32x16 sa = f32x16{};
#pragma unroll
          for (int k16 = 0; k16 < D / 32; ++k16) sa = qk16(sa, k16, qaop, sQa);
          const uint32_t am = range_bits(0, me.hiA, k0) >> (4 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((am >> acc_row(r, 0)) & 1u) sc[r] = sa[r];
        }
      }
      // the keys of this slice the lane's column sees; element r holds key
      // k0 + acc_row(r, g) = k0 + acc_row(r, 0) + 4 g
      const uint32_t cm =
          (me.valid ? range_bits(0, me.hiA, k0) | range_bits(me.loB, me.hiB, k0) : 0u) >> (4 * g);
      float smax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vis = (cm >> acc_row(r, 0)) & 1u;
        sc[r] = vis ? sc[r] * a.scale : -INFINITY;
        smax = fmaxf(smax, sc[r]);
      }
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      const float m_new = fmaxf(m, smax);
      const float alpha = expf(m - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = expf(sc[r] - m_new);  // 0 for a hidden key
        psum += pr;
        sP[acc_row(r, g) * 33 + l32] = pr;
      }
      psum += __shfl_xor(psum, 32, 64);
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    __syncthreads();
    if (act) {
      // P and V operands, read ahead of their MFMAs (V one O^T tile at a time)
      float pop[16];
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) pop[kk] = sP[(2 * kk + g) * 33 + l32];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float vop[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) vop[kk] = sV[(2 * kk + g) * LD + 32 * dt + l32];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop[kk], pop[kk], o[dt], 0, 0, 0);
      }
    }
  }

  // The waves' states (m, l, O^T over disjoint slices) merge exactly: wave
  // w > 0 leaves them in its own buffers, wave 0 rescales to the common max.
  if constexpr (NW > 1) {
    __syncthreads();
    if (w > 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sK[l32 * LD + 32 * dt + acc_row(r, g)] = o[dt][r];
      if (g == 0) {
        sP[l32] = m;
        sP[32 + l32] = l;
      }
    }
    __syncthreads();
    if (w > 0) return;
    for (int v = 1; v < NW; ++v) {
      const float* xo = sKw + v * 32 * LD;
      const float* xs = sPw + v * 32 * 33;
      const float mv = xs[l32], lv = xs[32 + l32];
      const float mn = fmaxf(m, mv);
      const float a0 = expf(m - mn), a1 = expf(mv - mn);
      l = l * a0 + lv * a1;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[dt][r] = o[dt][r] * a0 + xo[l32 * LD + 32 * dt + acc_row(r, g)] * a1;
    }
  }

  // O^T tile dt, element r of lane (l32, g): dimension 32 dt + acc_row(r, g) of column l32
  if (!me.valid) return;
  if (PHASE1) {
    float* op = a.o + ((s * a.L + me.row) * a.Hq + me.head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) op[32 * dt + acc_row(r, g)] = o[dt][r] / l;
  } else {
    const int64_t b = ((s * a.q_tokens + me.row) * a.Hq + me.head) * a.n_split + sigma;
    const bool any = l > 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        a.o_part[b * D + 32 * dt + acc_row(r, g)] = any ? o[dt][r] / l : 0.0f;
    if (g == 0) a.lse_part[b] = any ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// LSE merge: one workgroup per (sequence, query, head) row.
// ---------------------------------------------------------------------------
struct MergeArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse_out;
  int64_t rows;
  int32_t n_split, o_f32;
};

// One workgroup per (sequence, query, head) row. Thread t owns float4
// column t % (D/4) of the output and the splits i = t / (D/4) (mod SG): it
// loads their partials and log-sum-exps into registers at once, so the merge
// costs one round trip to memory; the split groups are summed through LDS.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a) {
  constexpr int C4 = D / 4;       // float4 columns of a row
  constexpr int SG = 256 / C4;    // split groups
  constexpr int U = 24;           // splits per thread and batch
  __shared__ float4 osum[SG][C4];
  __shared__ float zsum[SG];
  __shared__ float red[4];
  const int t = threadIdx.x, d4 = t % C4, sg = t / C4, lane = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.x;
  const int n = a.n_split;
  const float* lp = a.lse_part + row * n;
  const float4* op = (const float4*)(a.o_part + row * (int64_t)n * D);
  float4 ov[U];
  float lv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = sg + SG * u;
    ov[u] = i < n ? op[(int64_t)i * C4 + d4] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    lv[u] = i < n ? lp[i] : -INFINITY;
  }
  // m = max_s lse_s over every split (block reduction)
  float mx = -INFINITY;
  for (int i = t; i < n; i += 256) mx = fmaxf(mx, lp[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool empty = mx == -INFINITY;
  // this thread's share of z = sum_s exp(lse_s - m) and of sum_s exp(lse_s - m) o_s
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float z = 0.0f;
  if (!empty) {
    for (int i0 = 0; i0 < n; i0 += SG * U) {
      if (i0 > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + sg + SG * u;
          ov[u] = i < n ? op[(int64_t)i * C4 + d4] : float4{0.0f, 0.0f, 0.0f, 0.0f};
          lv[u] = i < n ? lp[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wgt = expf(lv[u] - mx);  // exp(-inf) = 0 past the last split
        z += wgt;
        acc.x = fmaf(wgt, ov[u].x, acc.x);
        acc.y = fmaf(wgt, ov[u].y, acc.y);
        acc.z = fmaf(wgt, ov[u].z, acc.z);
        acc.w = fmaf(wgt, ov[u].w, acc.w);
      }
    }
  }
  osum[sg][d4] = acc;
  if (d4 == 0) zsum[sg] = z;
  __syncthreads();
  if (t < C4) {
    float4 o = osum[0][t];
    float zt = zsum[0];
#pragma unroll
    for (int k = 1; k < SG; ++k) {
      o.x += osum[k][t].x;
      o.y += osum[k][t].y;
      o.z += osum[k][t].z;
      o.w += osum[k][t].w;
      zt += zsum[k];
    }
    const float inv = empty ? 0.0f : 1.0f / zt;
    const float v[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
    if (a.o_f32) {
      ((float4*)a.o)[row * C4 + t] = float4{v[0], v[1], v[2], v[3]};
    } else {
      uint2 b;
      b.x = pack_bf16(v[0], v[1]);
      b.y = pack_bf16(v[2], v[3]);
      ((uint2*)a.o)[row * C4 + t] = b;
    }
    if (t == 0 && a.lse_out) a.lse_out[row] = empty ? -INFINITY : mx + logf(zt);
  }
}

// The merge for many rows (a query step: n_query * Hq rows): one wave per
// row, so that a launch holds thousands of light waves and streams the
// partials at full bandwidth (the kernel above holds a row's splits in a
// workgroup's registers at once: one memory round trip, the right shape for
// the few rows of a decode step, but its registers cap how many workgroups a
// CU holds). Lane l takes float4 column l % C4 and the splits congruent to
// l / C4 modulo SPG = 64 / C4; the lanes of a column add their shares with
// two (D = 128) or three (D = 64) exchanges.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_rows_kernel(const MergeArgs a) {
  constexpr int C4 = D / 4;     // float4 columns of a row
  constexpr int SPG = 64 / C4;  // split groups in a wave
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int n = a.n_split;
  const float* lp = a.lse_part + row * n;
  const float4* op = (const float4*)(a.o_part + row * (int64_t)n * D);
  // m = max_s lse_s, z = sum_s exp(lse_s - m) (every lane takes splits lane, lane + 64, ...)
  float mx = -INFINITY;
  for (int i = lane; i < n; i += 64) mx = fmaxf(mx, lp[i]);
  mx = wave_max(mx);
  const bool empty = mx == -INFINITY;
  float z = 0.0f;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!empty) {
    for (int i = lane; i < n; i += 64) z += expf(lp[i] - mx);
    z = wave_sum(z);
    const int c = lane % C4;
    int i = lane / C4;
#pragma unroll 4
    for (; i < n; i += SPG) {
      const float wgt = expf(lp[i] - mx);  // exp(-inf) = 0 for an empty split
      const float4 v = op[(int64_t)i * C4 + c];
      acc.x = fmaf(wgt, v.x, acc.x);
      acc.y = fmaf(wgt, v.y, acc.y);
      acc.z = fmaf(wgt, v.z, acc.z);
      acc.w = fmaf(wgt, v.w, acc.w);
    }
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
      acc.x += __shfl_xor(acc.x, off, 64);
      acc.y += __shfl_xor(acc.y, off, 64);
      acc.z += __shfl_xor(acc.z, off, 64);
      acc.w += __shfl_xor(acc.w, off, 64);
    }
  }
  if (lane < C4) {
    const float inv = empty ? 0.0f : 1.0f / z;
    const float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    if (a.o_f32) {
      ((float4*)a.o)[row * C4 + lane] = float4{v[0], v[1], v[2], v[3]};
    } else {
      uint2 b;
      b.x = pack_bf16(v[0], v[1]);
      b.y = pack_bf16(v[2], v[3]);
      ((uint2*)a.o)[row * C4 + lane] = b;
    }
    if (lane == 0 && a.lse_out) a.lse_out[row] = empty ? -INFINITY : mx + logf(z);
  }
}

int check_launch() { return hipGetLastError() == hipSuccess ? STAR_OK : STAR_ERR_HIP; }

// Rows from which the merge takes one wave per row: four waves per CU.
constexpr int64_t kMergeRowsPerWave = 1024;

// kWideWaves (8 waves per wide-kernel workgroup): two per SIMD, 32 columns
// each (four waves of 64 columns need more than the 512 registers of a lane
// and spill).

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Every launcher refuses a grid that does not fit HIP's 32-bit count of
// work-items (grid_fits) with STAR_ERR_SHAPE before enqueueing it; the
// entry points have already checked every grid of the call.
template <bool PAGED, bool ROPE>
static int kv_write_impl(const Dims& d, void* kc, void* vc, int64_t pos0, const void* ks,
                         const void* vs, int64_t n_tok, const PageMap& pm, const float* rope_cos,
                         const float* rope_sin, void* stream) {
  KvArgs a;
  a.pm = pm;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.kc = kc;
  a.vc = vc;
  a.ks = ks;
  a.vs = vs;
  a.pos0 = pos0;
  a.n_tok = n_tok;
  a.rows = d.rows;
  a.t0 = pos0 / 64;
  a.nt = (int32_t)((pos0 + n_tok - 1) / 64 - a.t0 + 1);
  a.Hkv = d.Hkv;
  if (!grid_fits((int64_t)a.nt * d.B * d.Hkv, 256)) return STAR_ERR_SHAPE;
  const dim3 grid((unsigned)((int64_t)a.nt * d.B * d.Hkv));
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == STAR_BF16) {
    if (d.D == 128)
      hipLaunchKernelGGL((kv_write_kernel<uint16_t, 128, PAGED, ROPE>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_write_kernel<uint16_t, 64, PAGED, ROPE>), grid, dim3(256), 0, st, a);
  } else {
    if (d.D == 128)
      hipLaunchKernelGGL((kv_write_kernel<float, 128, PAGED, ROPE>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_write_kernel<float, 64, PAGED, ROPE>), grid, dim3(256), 0, st, a);
  }
  return check_launch();
}

int launch_kv_write(const Dims& d, void* kc, void* vc, int64_t pos0, const void* ks,
                    const void* vs, int64_t n_tok, void* stream, const int32_t* table,
                    int32_t maxp, const float* rope_cos, const float* rope_sin) {
  const PageMap pm{table, maxp};
  if (rope_cos)  // rotary embedding: the contiguous cache
    return kv_write_impl<false, true>(d, kc, vc, pos0, ks, vs, n_tok, pm, rope_cos, rope_sin,
                                      stream);
  return table ? kv_write_impl<true, false>(d, kc, vc, pos0, ks, vs, n_tok, pm, nullptr, nullptr,
                                            stream)
               : kv_write_impl<false, false>(d, kc, vc, pos0, ks, vs, n_tok, pm, nullptr, nullptr,
                                             stream);
}

static F32Args f32_args(const Dims& d, const void* kc, const void* vc, const void* q) {
  F32Args a{};
  a.k = (const float*)kc;
  a.v = (const float*)vc;
  a.q = (const float*)q;
  a.rows = d.rows;
  a.L = d.L;
  a.blk = d.blk;
  a.anc = d.anc;
  a.n_blocks = d.n_blocks;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.scale = d.scale;
  return a;
}

template <int ROPE>
static int phase1_impl(const Dims& d, const void* kc, const void* vc, const void* q, void* o,
                       const float* rope_cos, const float* rope_sin, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == STAR_F32) {
    F32Args a = f32_args(d, kc, vc, q);
    a.o = (float*)o;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.q_tokens = d.L;
    // the matrix cores: one workgroup per 32 context rows of a head
    if (!grid_fits(f32m_phase1_grid(d), 64 * f32m_waves(d.D))) return STAR_ERR_SHAPE;
    const dim3 grid((unsigned)f32m_phase1_grid(d));
    const dim3 block((unsigned)(64 * f32m_waves(d.D)));
    if (d.D == 128) hipLaunchKernelGGL((attn_f32m_kernel<128, true, false, ROPE>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_f32m_kernel<64, true, false, ROPE>), grid, block, 0, st, a);
    return check_launch();
  }
  WideArgs a{};
  a.k = (const uint16_t*)kc;
  a.v = (const uint16_t*)vc;
  a.q = (const uint16_t*)q;
  a.o = (uint16_t*)o;
  a.rows = d.rows;
  a.q_tokens = d.L;
  a.L = d.L;
  a.blk = d.blk;
  a.anc = d.anc;
  a.n_blocks = d.n_blocks;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  const WideGeom gm = phase1_geom(d);
  a.HW = d.HW;
  a.HQ = gm.HQ;
  a.BM = gm.BM;
  a.NG = gm.NG;
  a.NRT = gm.NRT;
  a.scale = d.scale;
  a.c2 = d.scale_log2;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  if (!grid_fits(gm.grid, 64 * kWideWaves)) return STAR_ERR_SHAPE;
  const dim3 grid((unsigned)gm.grid);
  if (d.D == 128)
    hipLaunchKernelGGL((attn_wide_kernel<128, kWideWaves, 8 / kWideWaves, true, false, ROPE, false>), grid,
                       dim3(64 * kWideWaves), 0, st, a);
  else
    hipLaunchKernelGGL((attn_wide_kernel<64, kWideWaves, 8 / kWideWaves, true, false, ROPE, false>), grid,
                       dim3(64 * kWideWaves), 0, st, a);
  return check_launch();
}

int launch_phase1(const Dims& d, const void* kc, const void* vc, const void* q, void* o,
                  void* stream, const float* rope_cos, const float* rope_sin, int rope_mode) {
  if (!rope_cos) return phase1_impl<kRopeNone>(d, kc, vc, q, o, nullptr, nullptr, stream);
  if (rope_mode == STAR_ROPE_ADJACENT)
    return phase1_impl<kRopeAdjacent>(d, kc, vc, q, o, rope_cos, rope_sin, stream);
  return phase1_impl<kRopeOriginal>(d, kc, vc, q, o, rope_cos, rope_sin, stream);
}

static DecodeArgs decode_args(const Dims& d, const Plan& p, const void* kc, const void* vc,
                              int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                              float* lse_part) {
  DecodeArgs a{};
  a.k = (const uint16_t*)kc;
  a.v = (const uint16_t*)vc;
  a.q = (const uint16_t*)q;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.rows = d.rows;
  a.L = d.L;
  a.blk = d.blk;
  a.kv_len = kv_len;
  a.n_query = n_query;
  a.wg_rows = p.wg_rows;
  a.bnd_period = p.bnd_period;
  a.n_split = p.n_split;
  a.n_blocks = d.n_blocks;
  a.n_wg = p.n_wg;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.NG = d.B * d.Hkv;
  (void)decode_grid(d, p, &a.WPG);
  a.scale = d.scale;
  a.c2 = d.scale_log2;
  return a;
}

template <bool FUSED, bool PAGED, bool MID>
static int launch_decode_mid(const Dims& d, const DecodeArgs& a, hipStream_t st) {
  if (!grid_fits((int64_t)a.NG * a.WPG, 256)) return STAR_ERR_SHAPE;
  const dim3 grid((unsigned)((int64_t)a.NG * a.WPG));
  if (d.D == 128)
    hipLaunchKernelGGL((attn_decode_kernel<128, FUSED, PAGED, MID>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<64, FUSED, PAGED, MID>), grid, dim3(256), 0, st, a);
  return STAR_OK;
}

template <bool FUSED, bool PAGED>
static int launch_decode(const Dims& d, const DecodeArgs& a, hipStream_t st) {
  // host boundaries (block starts, the context end) off the 32-key slice grid
  if (d.L % kSlice != 0 || d.blk % kSlice != 0) return launch_decode_mid<FUSED, PAGED, true>(d, a, st);
  return launch_decode_mid<FUSED, PAGED, false>(d, a, st);
}

template <bool PAGED>
static int phase2_partial_impl(const Dims& d, const Plan& p, const void* kc, const void* vc,
                               int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                               float* lse_part, const PageMap& pm, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == STAR_F32) {
    F32Args a = f32_args(d, kc, vc, q);
    a.pm = pm;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.q_tokens = n_query;
    a.kv_len = kv_len;
    a.blk_len = p.blk_len;
    a.tail_len = p.tail_len;
    a.per_block = p.per_block;
    a.n_split = p.n_split;
    // the matrix cores: one workgroup per 32 (query row, head) columns of a kv head and split
    const int64_t n = f32m_phase2_grid(d, p, n_query);
    if (!grid_fits(n, 64 * f32m_waves(d.D))) return STAR_ERR_SHAPE;
    const dim3 grid((unsigned)n);
    const dim3 block((unsigned)(64 * f32m_waves(d.D)));
    if (d.D == 128) hipLaunchKernelGGL((attn_f32m_kernel<128, false, PAGED, kRopeNone>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_f32m_kernel<64, false, PAGED, kRopeNone>), grid, block, 0, st, a);
    return check_launch();
  }
  if (p.narrow && p.balanced) {
    DecodeArgs a = decode_args(d, p, kc, vc, kv_len, q, n_query, o_part, lse_part);
    a.pm = pm;
    const int rc = launch_decode<false, PAGED>(d, a, st);
    return rc ? rc : check_launch();
  }
  if (p.narrow) {
    NarrowArgs a{};
    a.k = (const uint16_t*)kc;
    a.v = (const uint16_t*)vc;
    a.q = (const uint16_t*)q;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.rows = d.rows;
    a.L = d.L;
    a.blk = d.blk;
    a.kv_len = kv_len;
    a.n_query = n_query;
    a.blk_len = p.blk_len;
    a.tail_len = p.tail_len;
    a.per_block = p.per_block;
    a.n_split = p.n_split;
    a.n_blocks = d.n_blocks;
    a.Hq = d.Hq;
    a.Hkv = d.Hkv;
    a.G = d.G;
    a.NG = d.B * d.Hkv;
    a.scale = d.scale;
    a.c2 = d.scale_log2;
    a.pm = pm;
    if (!grid_fits((int64_t)a.NG * p.n_split, 256)) return STAR_ERR_SHAPE;
    const dim3 grid((unsigned)((int64_t)a.NG * p.n_split));
    if (d.D == 128)
      hipLaunchKernelGGL((attn_narrow_kernel<128, false, PAGED>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_narrow_kernel<64, false, PAGED>), grid, dim3(256), 0, st, a);
    return check_launch();
  }
  WideArgs a{};
  a.k = (const uint16_t*)kc;
  a.v = (const uint16_t*)vc;
  a.q = (const uint16_t*)q;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.rows = d.rows;
  a.q_tokens = n_query;
  a.L = d.L;
  a.blk = d.blk;
  a.anc = d.anc;
  a.kv_len = kv_len;
  a.blk_len = p.blk_len;
  a.tail_len = p.tail_len;
  a.per_block = p.per_block;
  a.n_split = p.n_split;
  a.n_blocks = d.n_blocks;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  const WideGeom gm = wide2_geom(d, p);
  a.HW = d.HW;
  a.HQ = gm.HQ;
  a.BM = gm.BM;
  a.NG = gm.NG;
  a.NRT = gm.NRT;
  a.scale = d.scale;
  a.c2 = d.scale_log2;
  a.pm = pm;
  if (!grid_fits(gm.grid, 64 * kWideWaves)) return STAR_ERR_SHAPE;
  const dim3 grid((unsigned)gm.grid);
  // one reader per split: a non-temporal stream; several: L2 serves the rest
  const bool kv_nt = a.HQ * a.NRT == 1;
  if (wide2_short(gm, n_query)) {
    if (d.D == 128 && kv_nt)
      hipLaunchKernelGGL((attn_wide_short_kernel<128, kWideWaves, PAGED, true>), grid,
                         dim3(64 * kWideWaves), 0, st, a);
    else if (d.D == 128)
      hipLaunchKernelGGL((attn_wide_short_kernel<128, kWideWaves, PAGED, false>), grid,
                         dim3(64 * kWideWaves), 0, st, a);
    else if (kv_nt)
      hipLaunchKernelGGL((attn_wide_short_kernel<64, kWideWaves, PAGED, true>), grid,
                         dim3(64 * kWideWaves), 0, st, a);
    else
      hipLaunchKernelGGL((attn_wide_short_kernel<64, kWideWaves, PAGED, false>), grid,
                         dim3(64 * kWideWaves), 0, st, a);
    return check_launch();
  }
  if (d.D == 128 && kv_nt)
    hipLaunchKernelGGL((attn_wide_kernel<128, kWideWaves, 8 / kWideWaves, false, PAGED, kRopeNone, true>),
                       grid, dim3(64 * kWideWaves), 0, st, a);
  else if (d.D == 128)
    hipLaunchKernelGGL((attn_wide_kernel<128, kWideWaves, 8 / kWideWaves, false, PAGED, kRopeNone, false>),
                       grid, dim3(64 * kWideWaves), 0, st, a);
  else if (kv_nt)
    hipLaunchKernelGGL((attn_wide_kernel<64, kWideWaves, 8 / kWideWaves, false, PAGED, kRopeNone, true>),
                       grid, dim3(64 * kWideWaves), 0, st, a);
  else
    hipLaunchKernelGGL((attn_wide_kernel<64, kWideWaves, 8 / kWideWaves, false, PAGED, kRopeNone, false>),
                       grid, dim3(64 * kWideWaves), 0, st, a);
  return check_launch();
}

int launch_phase2_partial(const Dims& d, const Plan& p, const void* kc, const void* vc,
                          int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                          float* lse_part, void* stream, const int32_t* table, int32_t maxp) {
  const PageMap pm{table, maxp};
  return table ? phase2_partial_impl<true>(d, p, kc, vc, kv_len, q, n_query, o_part, lse_part, pm,
                                           stream)
               : phase2_partial_impl<false>(d, p, kc, vc, kv_len, q, n_query, o_part, lse_part, pm,
                                            stream);
}

template <bool PAGED>
static int decode_step_impl(const Dims& d, const Plan& p, void* kc, void* vc, int64_t kv_len,
                            const void* q, const void* k_new, const void* v_new, int64_t n_query,
                            float* o_part, float* lse_part, const PageMap& pm, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.balanced) {
    DecodeArgs a = decode_args(d, p, kc, vc, kv_len, q, n_query, o_part, lse_part);
    a.k_new = (const uint16_t*)k_new;
    a.v_new = (const uint16_t*)v_new;
    a.pm = pm;
    const int rc = launch_decode<true, PAGED>(d, a, st);
    if (rc) return rc;
  } else {
    NarrowArgs a{};
    a.k = (const uint16_t*)kc;
    a.v = (const uint16_t*)vc;
    a.q = (const uint16_t*)q;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.rows = d.rows;
    a.L = d.L;
    a.blk = d.blk;
    a.kv_len = kv_len;
    a.n_query = n_query;
    a.blk_len = p.blk_len;
    a.tail_len = p.tail_len;
    a.per_block = p.per_block;
    a.n_split = p.n_split;
    a.n_blocks = d.n_blocks;
    a.Hq = d.Hq;
    a.Hkv = d.Hkv;
    a.G = d.G;
    a.NG = d.B * d.Hkv;
    a.scale = d.scale;
    a.c2 = d.scale_log2;
    a.k_new = (const uint16_t*)k_new;
    a.v_new = (const uint16_t*)v_new;
    a.pm = pm;
    if (!grid_fits((int64_t)a.NG * p.n_split, 256)) return STAR_ERR_SHAPE;
    const dim3 grid((unsigned)((int64_t)a.NG * p.n_split));
    if (d.D == 128)
      hipLaunchKernelGGL((attn_narrow_kernel<128, true, PAGED>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_narrow_kernel<64, true, PAGED>), grid, dim3(256), 0, st, a);
  }
  return check_launch();
}

int launch_decode_step(const Dims& d, const Plan& p, void* kc, void* vc, int64_t kv_len,
                       const void* q, const void* k_new, const void* v_new, int64_t n_query,
                       float* o_part, float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                       void* stream, const int32_t* table, int32_t maxp) {
  const PageMap pm{table, maxp};
  const int rc = table ? decode_step_impl<true>(d, p, kc, vc, kv_len, q, k_new, v_new, n_query,
                                                o_part, lse_part, pm, stream)
                       : decode_step_impl<false>(d, p, kc, vc, kv_len, q, k_new, v_new, n_query,
                                                 o_part, lse_part, pm, stream);
  if (rc) return rc;
  return launch_lse_merge(d, n_query, p.n_split, o_part, lse_part, o, o_dtype, lse_out, stream);
}

int launch_lse_merge(const Dims& d, int64_t n_query, int32_t n_split, const float* o_part,
                     const float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                     void* stream) {
  MergeArgs a;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.o = o;
  a.lse_out = lse_out;
  a.rows = (int64_t)d.B * n_query * d.Hq;
  a.n_split = n_split;
  a.o_f32 = o_dtype == STAR_F32;
  if (!grid_fits(a.rows, 256)) return STAR_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (a.rows >= kMergeRowsPerWave) {
    // many rows: one wave per row, four rows per workgroup
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    if (d.D == 128) hipLaunchKernelGGL((lse_merge_rows_kernel<128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((lse_merge_rows_kernel<64>), grid, dim3(256), 0, st, a);
    return check_launch();
  }
  const dim3 grid((unsigned)a.rows);
  if (d.D == 128) hipLaunchKernelGGL((lse_merge_kernel<128>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((lse_merge_kernel<64>), grid, dim3(256), 0, st, a);
  return check_launch();
}

// ---------------------------------------------------------------------------
// Scratch of star_attn_decode_step_noalloc: the split partials of one decode
// step, in a file-scope device array that every GPU the library runs on holds
// until the process ends. In host code `scratch` only names the symbol; its
// device address on the current GPU comes from hipGetSymbolAddress, looked up
// once per device (with that device current) and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[STAR_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; null until looked up
}  // namespace

int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return STAR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STAR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return STAR_OK;
}

}  // namespace star
