// Peak probe: a bf16 MFMA issue loop, so that the measurement reports the
// matrix-core rate this chip actually sustains beside the published peak.
// Not part of the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_peak.h"

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));

// Four accumulators, each fed two MFMAs back to back (the fastest issue order
// measured for v_mfma_f32_16x16x32_bf16 on gfx950); every wave of every
// workgroup runs `iters` rounds of 16 MFMAs and stores one sum per lane so that
// nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int32_t iters) {
  const int tid = threadIdx.x;
  bf16x8 a0, a1, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a0[e] = (__bf16)(tid * 1e-3f);
    a1[e] = (__bf16)(tid * 2e-3f);
    b[e] = (__bf16)(e * 0.5f);
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c0, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c1, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c3, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c3, 0, 0, 0);
    }
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  out[(int64_t)blockIdx.x * 256 + tid] = s[0] + s[1] + s[2] + s[3];
}

// HBM read probe: every thread streams 16-byte loads over the buffer
// (grid-stride) and stores one word, so the kernel moves `bytes` in and a
// negligible amount out.
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
__global__ __launch_bounds__(256) void read_loop_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                        uint32_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i = gid; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[gid] = acc;
}

}  // namespace

extern "C" int smla_peak_hbm_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* out, void* stream) {
  if (buf == nullptr || out == nullptr || bytes < 16 || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return 1;
  hipLaunchKernelGGL(read_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int smla_peak_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || out == nullptr) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" double smla_peak_mfma_flops(int32_t blocks, int32_t iters) {
  // 4 waves a workgroup, 16 MFMAs a round, 16 x 16 x 32 multiply-adds each
  return (double)blocks * 4.0 * (double)iters * 16.0 * (16.0 * 16.0 * 32.0 * 2.0);
}
