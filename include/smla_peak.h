/*
 * smla_peak.h -- C ABI of the peak probe built beside the decode library
 * (libsmla_peak.so).  Not part of the decode path: bench.py uses it to report
 * the bf16 matrix-core rate the chip sustains next to the published peak.
 */
#ifndef SMLA_PEAK_H
#define SMLA_PEAK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * smla_peak_mfma_bf16 -- enqueue `blocks` workgroups of 4 waves, each wave
 * running `iters` rounds of 16 v_mfma_f32_16x16x32_bf16 on register operands,
 * on `stream` (a hipStream_t).  `out` is a device buffer of blocks * 256 floats
 * owned by the caller (one sum per thread keeps the work from being removed).
 * Returns 0, 1 for a bad argument (nothing enqueued), or 5 if the launch failed.
 */
int smla_peak_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

/* smla_peak_mfma_flops -- the bf16 flops one such launch performs. */
double smla_peak_mfma_flops(int32_t blocks, int32_t iters);

/*
 * smla_peak_hbm_read -- enqueue a read of the first `bytes` (rounded down to a
 * multiple of 16) of the 16-byte aligned device buffer `buf` by `blocks`
 * workgroups of 256 threads in 16-byte loads; every thread stores one word to
 * `out`, a device buffer of blocks * 256 uint32 owned by the caller.  Returns 0,
 * 1 for a bad argument (nothing enqueued), or 5 if the launch failed.
 */
int smla_peak_hbm_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_PEAK_H */
