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
  int32_t col_parts;          // workgroups per job: 1 to 16 for 64 heads, else (h_q / 16) x 1, 2 or 4; 1 for a direct FP8 output
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

// One launch of the FP8 prefill attention and its combine.  Device pointers only.
struct PrefillArgs {
  const uint8_t* q;           // [B][Sq][h_q][128] e4m3 codes
  const uint8_t* k;           // [B][Skv][h_kv][128]
  const uint8_t* v;           // [B][Skv][h_kv][128]
  const int32_t* seqlen_q;    // [B]
  const int32_t* seqlen_kv;   // [B]
  const float* sink;          // [h_q] or nullptr
  float* o_part;              // [S][B][Sq][h_q][128] (split mode)
  float* lse_part;            // [S][B][Sq][h_q]      (split mode)
  void* out;                  // [B][Sq][h_q][128] bf16 / f32, or nullptr
  float* lse_out;             // [B][Sq][h_q] or nullptr
  float* amax_out;            // one float or nullptr
  int32_t batch, h_q, h_kv, sq_max, skv_max, num_splits, n_tiles;
  int32_t causal, out_dtype;
  float scale_log2;           // softmax_scale * descale_q * descale_k * log2(e)
  float descale_v;
  int32_t n_work;             // batch * num_splits * n_tiles * h_q workgroups of the attention launch
  int32_t cus;
};

// Each returns the launch status (hipSuccess or the runtime's error).
hipError_t launch_decode_partial(const DecodeArgs& a, bool kv_fp8, hipStream_t stream);
hipError_t launch_decode_direct(const DecodeArgs& a, bool kv_fp8, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// FP8 prefill: split (partials) or direct attention; then (out given) the combine.
hipError_t launch_prefill(const PrefillArgs& a, bool split, hipStream_t stream);
hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t stream);

// Device address of the current device's copy of the no-allocation entry
// point's scratch (SMLA_NOALLOC_SCRATCH_BYTES); looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace smla
