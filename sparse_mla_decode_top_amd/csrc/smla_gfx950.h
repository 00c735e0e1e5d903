// gfx950 (CDNA4) device primitives shared by the library's kernels: vector
// types, direct-to-LDS loads, LDS barriers, wave reductions on DPP and the row
// swaps, bf16 and f16 packing and exact e4m3 -> bf16 / f16 conversion.  Device
// code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef float f32x2 __attribute__((__vector_size__(8)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte direct-to-LDS load per lane: segment O of a row, i.e. global
// address src + O * GSTEP and LDS address lds_base + O * LSTEP + 16 * lane (the
// instruction offset O * GSTEP is added to both addresses, so m0 takes
// lds_base + O * (LSTEP - GSTEP)).  Lets a block's gather be spread over the
// MFMA work of the previous block.
template <int LSTEP, int GSTEP, int O>
__device__ __forceinline__ void dma_one(const void* src, uint32_t lds_base_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off offset:%4\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base_uniform), "n"(O * (LSTEP - GSTEP)), "n"(O * GSTEP)
      : "memory");
}

// Hides a value from the optimiser, so that an address computed from it inside
// the loop keeps its constant parts as instruction offsets instead of being
// hoisted as many loop-invariant registers.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that only drains LDS traffic (in-flight tile prefetches
// keep running across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Butterfly reductions of a whole wave without LDS round trips: DPP swaps
// inside each 16-lane row (lane ^ 1, ^ 2, then the 8- and 16-lane mirrors),
// then the row swaps below.  Every lane ends with the same value: each step
// combines two equal-shaped partial results with a commutative operation.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap moves: each swap hands every lane the value of its
// partner row, with no LDS round trip.
__device__ __forceinline__ float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));        // quad_perm [1,0,3,2]: lane ^ 1
  v = fmaxf(v, dpp<0x4E>(v));        // quad_perm [2,3,0,1]: lane ^ 2
  v = fmaxf(v, dpp<0x141>(v));       // row_half_mirror: the other quad of the 8 lanes
  v = fmaxf(v, dpp<0x140>(v));       // row_mirror: the other 8 lanes of the row
  return rows_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp<0xB1>(v);
  v = v + dpp<0x4E>(v);
  v = v + dpp<0x141>(v);
  v = v + dpp<0x140>(v);
  return rows_sum(v);
}

// Eight e4m3fn codes (two dwords, code k in byte k) as bf16 (exact for every code).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 w) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, o);
}

// Eight e4m3fn codes as f16 (exact for every code: e4m3 values are f16 values).
__device__ __forceinline__ f16x8 e4m3x8_to_f16(u32x2 w) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true));
  return __builtin_bit_cast(f16x8, o);
}

// Two floats as packed f16 (round to nearest even), `lo` in the low half: one
// v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, f16x2v));
}

// Two floats as packed bf16 (round to nearest even), `lo` in the low half: one
// v_cvt_pk_bf16_f32 (two scalar conversions would take two and a merge).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

}  // namespace smla
