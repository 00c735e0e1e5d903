// Internal interface between the C-ABI layer (smla_api.cpp) and the HIP
// kernels (smla_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

// Everything one launch of the attention kernel needs.  Device pointers only.
struct DecodeArgs {
  const uint16_t* q;          // [s_q][h_q][576] bf16 bits
  const uint8_t* kv;          // pool base address (bytes)
  const float* kv_scale;      // [n_pool] (FP8 pool) or nullptr
  const int32_t* indices;     // [s_q][topk]
  const float* sink;          // [h_q] or nullptr
  float* o_accum;             // [S][s_q][h_q][512]   (partial mode)
  float* lse_accum;           // [S][s_q][h_q]        (partial mode)
  void* out;                  // [s_q][h_q][512]      (direct mode)
  float* out_scale;           // [s_q] FP8 out: the scale (direct mode), or set to -0.0 for the combine
                              // (split mode with an FP8 output to follow); else nullptr
  float* lse_out;             // [s_q][h_q] or nullptr (direct mode)
  int64_t n_pool;
  int64_t row_stride_bytes;
  int32_t s_q, h_q, topk, num_splits, n_blocks;
  int32_t out_dtype;          // smla_out_dtype (direct mode)
  float scale_log2;           // softmax_scale * log2(e)
  int32_t col_parts;          // 1, 2, 4 or 8 workgroups per job, each owning 512 / col_parts output columns
  int32_t cus;                // compute units of the device (the launch plan's round size)
};

struct CombineArgs {
  const float* o_accum;
  const float* lse_accum;
  const float* sink;
  void* out;
  float* out_scale;
  float* lse_out;
  int32_t s_q, h_q, num_splits;
  int32_t out_dtype;
  int32_t heads_per_wg;       // bf16 / f32 output: -1 a quarter of a row per wave, 0 half a row, 4 four rows
                              // per workgroup
  int32_t scale_ready;        // FP8 output: out_scale and the token counters already seeded (by the attention
                              // kernel)
  int32_t cus;                // compute units of the device (the FP8 one-launch combine fits one round)
};

// Each returns the launch status (hipSuccess or the runtime's error).
hipError_t launch_decode_partial(const DecodeArgs& a, bool kv_fp8, hipStream_t stream);
hipError_t launch_decode_direct(const DecodeArgs& a, bool kv_fp8, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// Device address of the current device's copy of the no-allocation entry
// point's scratch (SMLA_NOALLOC_SCRATCH_BYTES); looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace smla
