/*
 * star_peaks.h - peak probes for MI355X (gfx950), libstarpeaks.so.
 *
 * Measurement tools, not part of the attention path: they measure what the
 * chip sustains on the three resources the attention kernels are bound by,
 * so that a kernel's rate can be read against the measured peak as well as
 * the published one (2.5 PFLOP/s dense bf16 MFMA at 2.4 GHz, 8 TB/s HBM).
 * The pages describe no kernel and print no hardware figure; these probes
 * belong to the measurement method, not to the method of the pages.
 *
 * Each entry point validates its arguments, launches its probe kernel once
 * to warm up and then `reps` times between two HIP events on `stream`, waits
 * for the stream, and writes the mean rate over the timed launches. Unlike
 * libstarattn they synchronise the stream. They allocate nothing: `sink` is
 * a caller-owned device buffer of at least STAR_PEAK_SINK_BYTES that the
 * probes only write if their result is a value that cannot occur (it keeps
 * the work from being optimised away). The grids fill all 256 CUs, one
 * workgroup each. Status codes are those of star_attn.h (STAR_OK,
 * STAR_ERR_INVALID_ARG before any launch, STAR_ERR_HIP on a HIP error).
 */
#ifndef STAR_PEAKS_H
#define STAR_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STAR_PEAK_SINK_BYTES 4096

/*
 * star_peak_mfma_bf16 - sustained v_mfma_f32_32x32x16_bf16 rate: 8 waves per
 * CU, each issuing `iters` x 4 MFMAs on four independent accumulators with
 * register operands (32768 FLOP each). *tflops = FLOP / mean launch time.
 * iters >= 1; reps >= 1.
 */
int star_peak_mfma_bf16(int32_t iters, int32_t reps, void* sink, double* tflops, void* stream);

/*
 * star_peak_hbm_read - HBM read rate of a non-temporal 16-byte-per-lane
 * stream: 4 waves per CU, each reading its own contiguous range of `buf`
 * (double-buffered, 16 loads of 1 KB in flight per wave). The first
 * *bytes_read bytes of buf are read (bytes rounded down to whole 16 KB
 * chunks per wave; at least 16 MiB). *gbs = bytes read / mean launch time.
 * buf: device memory of `bytes` bytes, read only.
 */
int star_peak_hbm_read(const void* buf, size_t bytes, int32_t reps, void* sink, double* gbs,
                       size_t* bytes_read, void* stream);

/*
 * star_peak_exp - v_exp_f32 rate: 8 waves per CU, each lane running 8
 * independent exp2 chains of `iters` steps. *gexp = exps per ns (G/s).
 */
int star_peak_exp(int32_t iters, int32_t reps, void* sink, double* gexp, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STAR_PEAKS_H */
