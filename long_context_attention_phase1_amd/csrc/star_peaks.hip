// Peak probes of libstarpeaks.so (include/star_peaks.h): the sustained bf16
// MFMA rate, the HBM read rate of a non-temporal stream and the v_exp_f32
// rate on gfx950, against which the attention kernels' rates are read beside
// the published peaks. Measurement tools; not part of the attention path.
#include <hip/hip_runtime.h>

#include "../../include/star_attn.h"
#include "../../include/star_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCUs = 256;          // one workgroup per CU
constexpr int kMfmaWaves = 8;      // two waves per SIMD, as the phase-1 kernel
constexpr int kStreamWaves = 4;    // one wave per SIMD, as the decode kernel
constexpr int kStreamU = 16;       // 1 KB loads per wave per buffer

// Four independent accumulation chains per wave keep the matrix pipe fed
// without operand traffic: the rate is the pipe's at the clock it holds.
__global__ __launch_bounds__(64 * kMfmaWaves) void peak_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.002f * (float)(lane - i));
    b[i] = (__bf16)(0.001f * (float)(lane + i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 1234.5f) sink[threadIdx.x] = s;  // never: keeps the chains live
}

// Each wave reads its own contiguous range of per_wave16 16-byte chunks with
// non-temporal loads, two buffers of kStreamU loads in flight.
__global__ __launch_bounds__(64 * kStreamWaves) void peak_stream_kernel(const u32x4* __restrict__ src,
                                                                       int64_t per_wave16,
                                                                       uint32_t* sink) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const u32x4* p = src + ((int64_t)blockIdx.x * kStreamWaves + w) * per_wave16 + lane;
  const int nchunk = (int)(per_wave16 / (64 * kStreamU));
  u32x4 x[kStreamU], y[kStreamU];
  uint32_t acc = 0;
  auto load = [&](u32x4 (&r)[kStreamU], int c) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u)
      r[u] = __builtin_nontemporal_load(p + ((int64_t)c * kStreamU + u) * 64);
  };
  auto eat = [&](const u32x4 (&r)[kStreamU]) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  };
  load(x, 0);
  for (int c = 0; c < nchunk; c += 2) {
    if (c + 1 < nchunk) load(y, c + 1);
    eat(x);
    if (c + 1 >= nchunk) break;
    if (c + 2 < nchunk) load(x, c + 2);
    eat(y);
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;  // never: keeps the loads live
}

// Eight independent chains x <- 2^(-x) per lane (bounded in (0, 1]; the
// negation is an input modifier of v_exp_f32, so the loop is exps only).
__global__ __launch_bounds__(64 * kMfmaWaves) void peak_exp_kernel(int iters, float* sink) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.01f * (float)(threadIdx.x & 63) + 0.1f * (float)k;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  if (s == 1234.5f) sink[threadIdx.x] = s;  // never
}

// Warm-up launch, then `reps` launches between two events; mean ms per launch.
template <typename F>
int time_launches(F launch, int reps, hipStream_t st, double* ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = STAR_ERR_HIP;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    launch();
    if (hipGetLastError() == hipSuccess && hipEventRecord(e0, st) == hipSuccess) {
      for (int r = 0; r < reps; ++r) launch();
      float t = 0.0f;
      if (hipGetLastError() == hipSuccess && hipEventRecord(e1, st) == hipSuccess &&
          hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&t, e0, e1) == hipSuccess) {
        *ms = (double)t / reps;
        rc = *ms > 0.0 ? STAR_OK : STAR_ERR_HIP;
      }
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return rc;
}

}  // namespace

extern "C" {

int star_peak_mfma_bf16(int32_t iters, int32_t reps, void* sink, double* tflops, void* stream) {
  if (iters < 1 || reps < 1 || !sink || !tflops) return STAR_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  double ms = 0.0;
  const int rc = time_launches(
      [&] {
        hipLaunchKernelGGL(peak_mfma_kernel, dim3(kCUs), dim3(64 * kMfmaWaves), 0, st, iters,
                           (float*)sink);
      },
      reps, st, &ms);
  if (rc) return rc;
  const double flop = (double)kCUs * kMfmaWaves * iters * 4.0 * (32.0 * 32.0 * 16.0 * 2.0);
  *tflops = flop / (ms * 1e-3) / 1e12;
  return STAR_OK;
}

int star_peak_hbm_read(const void* buf, size_t bytes, int32_t reps, void* sink, double* gbs,
                       size_t* bytes_read, void* stream) {
  const size_t chunk = (size_t)64 * kStreamU * 16;  // one buffer of one wave
  const size_t waves = (size_t)kCUs * kStreamWaves;
  if (!buf || !sink || !gbs || !bytes_read || reps < 1) return STAR_ERR_INVALID_ARG;
  if (bytes < ((size_t)16 << 20)) return STAR_ERR_INVALID_ARG;
  const size_t per_wave = bytes / waves / chunk * chunk;  // whole chunks, inside buf
  hipStream_t st = (hipStream_t)stream;
  double ms = 0.0;
  const int rc = time_launches(
      [&] {
        hipLaunchKernelGGL(peak_stream_kernel, dim3(kCUs), dim3(64 * kStreamWaves), 0, st,
                           (const u32x4*)buf, (int64_t)(per_wave / 16), (uint32_t*)sink);
      },
      reps, st, &ms);
  if (rc) return rc;
  *bytes_read = per_wave * waves;
  *gbs = (double)*bytes_read / (ms * 1e-3) / 1e9;
  return STAR_OK;
}

int star_peak_exp(int32_t iters, int32_t reps, void* sink, double* gexp, void* stream) {
  if (iters < 1 || reps < 1 || !sink || !gexp) return STAR_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  double ms = 0.0;
  const int rc = time_launches(
      [&] {
        hipLaunchKernelGGL(peak_exp_kernel, dim3(kCUs), dim3(64 * kMfmaWaves), 0, st, iters,
                           (float*)sink);
      },
      reps, st, &ms);
  if (rc) return rc;
  const double n = (double)kCUs * 64 * kMfmaWaves * iters * 8.0;
  *gexp = n / (ms * 1e-3) / 1e9;
  return STAR_OK;
}

}  // extern "C"
