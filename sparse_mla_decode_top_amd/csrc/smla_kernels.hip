// HIP kernels for split-KV sparse MLA decode on MI355X (gfx950, CDNA4).
//
// The operation follows FlashMLA PR #25 ("What changes": (query token, KV
// split) jobs, each walking its own block range and writing an fp32 partial
// normalised by its own denominator plus a log2-space LSE), "The Split-K
// Dispatch" ("The LSE Combine Strategy": merge with exp2 weights relative to
// the largest LSE) and cudnn-frontend PR #768 (near-equal block ranges with
// the remainder on the leading splits; an empty split is O = 0, LSE = -inf).
//
// decode kernel: one workgroup of 4 wave64s per (token, split) job.
//   * The 64 slots of a KV block share one tile: the index-driven gather copies
//     each selected 1152-byte row into LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4), double-buffered so block b+1 streams in while
//     block b is computed.  Masked slots are never read; their tile rows are
//     zero-filled.
//   * Wave w = 2*hg + x owns heads [32hg, 32hg+32).  For QK^T it takes slots
//     [32x, 32x+32) of the block: S^T[slot][head] = K . Q^T with
//     v_mfma_f32_32x32x16_bf16 (K from LDS, Q resident in VGPRs), so every lane
//     holds scores of exactly one head.  For PV it takes value columns
//     [256x, 256x+256): O^T[col][head] = V^T . P^T, the V^T operand read with
//     the gfx950 LDS transpose load ds_read_b64_tr_b16 from the same row-major
//     tile, so again every accumulator lane belongs to one head.
//   * Online softmax in log2 units with an integer running maximum M: each
//     weight is p = 2^(t - floor t) * 2^(floor t - M).  Its bf16 rounding does
//     not depend on M, and every rescale is an exact power of two, so the
//     partials of different split counts combine to the same value up to fp32
//     summation order.  The denominator sums the unrounded fp32 weights.
//   * P enters the PV product as two bf16 terms, hi = bf16(p) and
//     lo = bf16(p - hi), sharing each V^T operand: a bf16-rounded P alone
//     leaves O errors near 4e-3 when a few slots dominate (one 64-slot block);
//     hi + lo carries p to about 2^-17 relative.
//
// combine kernel: one thread per 4 output columns of a (token, head), reading
// the split-major partials.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((__vector_size__(64)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 64;                         // slots per KV block
constexpr int kRowChunks = 72;                   // 16-byte chunks per bf16 row (576 x 2 B)
constexpr int kTileChunks = kBlk * kRowChunks;   // 4608
constexpr int kTileBytes = kTileChunks * 16;     // 73728
constexpr int kCodeRowChunks = 36;               // 16-byte chunks per FP8 row (576 B)
constexpr int kCodeTileBytes = kBlk * kCodeRowChunks * 16;   // 36864
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

enum OutDtype { kOutBf16 = 0, kOutF32 = 1, kOutFp8 = 2 };

// ---------------------------------------------------------------------------
// LDS tile layout ("chunk-major").  A bf16 KV row is 72 chunks of 16 bytes
// (8 elements).  Chunk c of tile row r lives at chunk position
//     c * 64 + (r ^ 4 * (c & 3)),
// i.e. the 64 rows of one chunk column are contiguous.  Consequences:
//   * gather: one direct-to-LDS load instruction fills one chunk column, lane l
//     loading row l ^ 4(c & 3); wave w owns the columns c = w (mod 4), so each
//     lane gathers from ONE pool row at immediate offsets 16c;
//   * QK^T reads (32 rows x one chunk per 32 lanes) hit 32 consecutive
//     positions: conflict-free;
//   * PV transpose reads (4 rows x 2 adjacent chunks per 16 lanes): the XOR on
//     row bits 2..3 moves the two chunks to different bank halves.
// The FP8 code tile uses the same formula over its 36 chunks per row.
// ---------------------------------------------------------------------------
constexpr int kLoadsBf16 = kRowChunks / kWaves;          // 18 chunk columns per wave
constexpr int kLoadsFp8 = kCodeRowChunks / kWaves;       // 9
constexpr float kRescaleSlack = 8.0f;    // the running max only moves when exceeded by this

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS gather of one lane's row: N loads of 16 bytes at global offsets
// 64j (chunk columns w, w+4, ...) into LDS bytes base + 4096j + 16*lane (4 chunk
// columns apart).  The hardware adds the instruction offset to BOTH addresses
// (LDS address = m0 + offset + 16*lane), so m0 steps by 4096 - 64 = 4032 to
// land each load 4096 bytes after the previous one.  Issued as one inline-assembly
// block so that the compiler neither interleaves other m0 users nor inserts a
// vmcnt wait in front of the LDS reads of the other buffer (it cannot tell the
// prefetch buffer from the one being read); the kernel waits explicitly.  m0
// is saved and restored; one wait state follows each m0 write.
#define SMLA_DMA_STEP(OFF) \
  "s_add_u32 m0, m0, 4032\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:" #OFF "\n\t"
template <int N>
__device__ __forceinline__ void dma_row(const void* gptr, uint32_t lds_base_uniform);
template <>
__device__ __forceinline__ void dma_row<18>(const void* gptr, uint32_t lds_base_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      SMLA_DMA_STEP(64) SMLA_DMA_STEP(128) SMLA_DMA_STEP(192) SMLA_DMA_STEP(256)
      SMLA_DMA_STEP(320) SMLA_DMA_STEP(384) SMLA_DMA_STEP(448) SMLA_DMA_STEP(512)
      SMLA_DMA_STEP(576) SMLA_DMA_STEP(640) SMLA_DMA_STEP(704) SMLA_DMA_STEP(768)
      SMLA_DMA_STEP(832) SMLA_DMA_STEP(896) SMLA_DMA_STEP(960) SMLA_DMA_STEP(1024)
      SMLA_DMA_STEP(1088)
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base_uniform)
      : "memory");
}
template <>
__device__ __forceinline__ void dma_row<9>(const void* gptr, uint32_t lds_base_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      SMLA_DMA_STEP(64) SMLA_DMA_STEP(128) SMLA_DMA_STEP(192) SMLA_DMA_STEP(256)
      SMLA_DMA_STEP(320) SMLA_DMA_STEP(384) SMLA_DMA_STEP(448) SMLA_DMA_STEP(512)
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base_uniform)
      : "memory");
}
#undef SMLA_DMA_STEP

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that only drains LDS traffic (in-flight tile prefetches
// keep running across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Bit s of the result = bit (s ^ 4w) of m: undoes the lane <-> slot XOR of
// the gather assignment (xor 4 swaps nibbles, xor 8 swaps bytes).
__device__ __forceinline__ uint64_t unswizzle_mask(uint64_t m, int w) {
  if (w & 1) m = ((m & 0x0F0F0F0F0F0F0F0Full) << 4) | ((m >> 4) & 0x0F0F0F0F0F0F0F0Full);
  if (w & 2) m = ((m & 0x00FF00FF00FF00FFull) << 8) | ((m >> 8) & 0x00FF00FF00FF00FFull);
  return m;
}

// e4m3fn code of a finite fp32 value, round to nearest even, saturating at
// +-448, sign kept (also for values that round to zero).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling; RNE; 8 -> smallest normal
  } else {
    const uint32_t ab = __float_as_uint(a);
    const uint32_t e = (ab >> 23) - 127u + 7u;      // biased e4m3 exponent, 1..15
    const uint32_t m = ab & 0x7FFFFFu;
    uint32_t m3 = m >> 20;
    const uint32_t rem = m & 0xFFFFFu;
    m3 += (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
    code = (e << 3) + m3;                            // a carry moves into the exponent
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Job decode shared by every wave: blockIdx.x = token * num_splits + split.
// Blocks [b0, b1) of split s: near-equal ranges, the remainder on the leading
// splits, empty past the end.
struct Job {
  int t, s, b0, b1;
};
__device__ __forceinline__ Job decode_job(int num_splits, int n_blocks) {
  Job j;
  j.t = blockIdx.x / num_splits;
  j.s = blockIdx.x - j.t * num_splits;
  const int base = n_blocks / num_splits, rem = n_blocks - base * num_splits;
  j.b0 = j.s * base + min(j.s, rem);
  j.b1 = j.b0 + base + (j.s < rem ? 1 : 0);
  return j;
}

// ---------------------------------------------------------------------------
// The attention kernel.  KV_FP8: pool rows are e4m3 codes + a row scale.
// DIRECT: single-split job writing the final output (sink + cast fused).
// ---------------------------------------------------------------------------
template <bool KV_FP8, bool DIRECT>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  // LDS: two bf16 tiles (bf16 pool) or two code tiles + one bf16 tile (FP8
  // pool), the P exchange area and small reduction arrays.
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[kWaves * 2 * 64 * 16];
  __shared__ float s_max[2][64];
  __shared__ float s_l[2][64];
  __shared__ float s_scale[2][kBlk];
  __shared__ float s_red[kWaves];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;            // k-group of the MFMA operand layout
  const int hg = wave >> 1;           // head tile: heads [32hg, 32hg + 32)
  const int x = wave & 1;             // QK slot half / PV column half
  const int hh = 32 * hg + (lane & 31);   // this lane's head (MFMA column)
  const int partner = wave ^ 1;
  const int gslot = lane ^ (4 * wave);    // slot of the block whose row this lane gathers

  const Job job = decode_job(a.num_splits, a.n_blocks);
  const int t = job.t;
  const int32_t* idx_row = a.indices + (int64_t)t * a.topk;

  float M_run = kNegInf;              // integer-valued running max (log2 units)
  float l_run = 0.f;                  // this lane's share of the denominator
  f32x16 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[ct][i] = 0.f;

  if (job.b0 < job.b1) {
    auto load_idx = [&](int b) -> int {
      const int slot = b * kBlk + gslot;
      return (b < job.b1 && slot < a.topk) ? __builtin_nontemporal_load(idx_row + slot) : -1;
    };
    auto valid_of = [&](int idx) -> bool { return idx >= 0 && (int64_t)idx < a.n_pool; };
    int idx_cur = load_idx(job.b0);
    int idx_nxt = load_idx(job.b0 + 1);

    // Q fragments of this lane's head: B operand of S^T = K . Q^T.
    bf16x8 qf[36];
    {
      const bool hv = hh < a.h_q;
      const uint16_t* qrow = a.q + ((int64_t)t * a.h_q + (hv ? hh : 0)) * 576 + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + 16 * ks);
        if (!hv) v = u32x4{0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    const uint32_t tile_lds0 = lds_addr(s_tile);
    constexpr int kBufBytes = KV_FP8 ? kCodeTileBytes : kTileBytes;
    constexpr int kLoads = KV_FP8 ? kLoadsFp8 : kLoadsBf16;

    // Gather of one block into buffer `buf`: this lane's row, chunk columns
    // c = wave + 4j.  Masked slots are zero-filled, never read.
    auto issue_gather = [&](int idx_lane, int buf) {
      if (valid_of(idx_lane)) {
        const uint8_t* src = a.kv + (int64_t)idx_lane * a.row_stride_bytes + 16 * wave;
        dma_row<kLoads>(src, __builtin_amdgcn_readfirstlane(tile_lds0 + buf * kBufBytes + wave * 1024));
      } else {
        uint8_t* dst = s_tile + buf * kBufBytes + wave * 1024 + lane * 16;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) *(u32x4*)(dst + 4096 * j) = u32x4{0u, 0u, 0u, 0u};
      }
    };

    // ---- prologue: block b0 in flight ------------------------------------
    uint64_t vmask_cur = unswizzle_mask(__ballot(valid_of(idx_cur)), wave);
    issue_gather(idx_cur, 0);
    float sc_cur = (KV_FP8 && wave == 0 && valid_of(idx_cur)) ? a.kv_scale[idx_cur] : 0.f;
    const float scale_log2 = a.scale_log2;

    for (int b = job.b0; b < job.b1; ++b) {
      const int cur = (b - job.b0) & 1;
      wait_vmem_all();          // this wave's share of block b has landed
      lds_barrier();            // ... and every other wave's; block b-1 fully consumed

      // Prefetch block b+1 (its indices were loaded one block ahead).
      uint64_t vmask_nxt = 0;
      float sc_nxt = 0.f;
      if (b + 1 < job.b1) {
        vmask_nxt = unswizzle_mask(__ballot(valid_of(idx_nxt)), wave);
        issue_gather(idx_nxt, cur ^ 1);
        if (KV_FP8 && wave == 0 && valid_of(idx_nxt)) sc_nxt = a.kv_scale[idx_nxt];
      }
      const int idx_after = load_idx(b + 2);

      const uint8_t* tile;
      if (!KV_FP8) {
        tile = s_tile + cur * kTileBytes;
      } else {
        // Expand block b's e4m3 codes into the bf16 tile (exact) and publish
        // the row scales.  Wave w converts bf16 chunk columns c = w + 4j.
        uint8_t* btile = s_tile + 2 * kCodeTileBytes;
        const uint8_t* ctile = s_tile + cur * kCodeTileBytes;
        if (wave == 0) s_scale[cur][lane] = sc_cur;
        const int r = gslot;                       // row of bf16 position c*64 + lane
#pragma unroll 6
        for (int j = 0; j < kLoadsBf16; ++j) {
          const int c = wave + 4 * j;
          const int cc = c >> 1;                   // code chunk holding bf16 chunk c
          const u32x2 codes =
              *(const u32x2*)(ctile + (cc * 64 + (r ^ (4 * (cc & 3)))) * 16 + (c & 1) * 8);
          // v_cvt_scalef32_pk_bf16_fp8 with scale 1 is exact for every e4m3fn code.
          u32x4 o;
          o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], 1.0f, false));
          o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], 1.0f, true));
          o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], 1.0f, false));
          o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], 1.0f, true));
          *(u32x4*)(btile + (c * 64 + lane) * 16) = o;
        }
        lds_barrier();
        tile = btile;
      }

      // ---- S^T = K . Q^T over this wave's 32 slots --------------------------
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      {
        const int r = 32 * x + (lane & 31);
        // chunk c = 2ks + g sits at c*64 + (r ^ 4(c & 3)), c & 3 = 2(ks & 1) + g
        const uint8_t* kb0 = tile + g * 1024 + ((r ^ (4 * g)) * 16);
        const uint8_t* kb1 = tile + g * 1024 + ((r ^ (8 + 4 * g)) * 16);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(((ks & 1) ? kb1 : kb0) + 2048 * ks);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
        }
      }

      // ---- online softmax (log2 units, integer running max) -----------------
      float tv[16];
      float mloc = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = 32 * x + 8 * (i >> 2) + 4 * g + (i & 3);
        const bool v = (vmask_cur >> slot) & 1ull;
        float sv = sacc[i] * scale_log2;
        if (KV_FP8) sv *= s_scale[cur][slot];
        tv[i] = v ? sv : kNegInf;
        mloc = fmaxf(mloc, tv[i]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      if (lane < 32) s_max[x][hh] = mloc;
      lds_barrier();
      const float mblk = fmaxf(s_max[0][hh], s_max[1][hh]);
      float M_new = M_run;
      if (mblk != kNegInf && (M_run == kNegInf || mblk > M_run + kRescaleSlack)) M_new = floorf(mblk);
      const bool moved = (M_run != kNegInf) && (M_new != M_run);
      if (__any(moved)) {       // rare: rescale by an exact power of two
        const float alpha = moved ? __builtin_amdgcn_ldexpf(1.0f, (int)fmaxf(M_run - M_new, -200.f)) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[ct][i] *= alpha;
      }
      M_run = M_new;

      uint32_t pk[8], pl[8];      // bf16 pairs of p: high part, low part
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float pv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float tt = tv[i + u];
          float p = 0.f;
          if (tt != kNegInf) {
            const float fl = floorf(tt);
            p = __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(tt - fl), (int)fmaxf(fl - M_new, -200.f));
          }
          psum += p;
          if (KV_FP8) {
            const int slot = 32 * x + 8 * ((i + u) >> 2) + 4 * g + ((i + u) & 3);
            p *= s_scale[cur][slot];
          }
          pv[u] = p;
        }
        pk[i >> 1] = pack_bf16x2(pv[0], pv[1]);
        const float h0 = __uint_as_float(pk[i >> 1] << 16), h1 = __uint_as_float(pk[i >> 1] & 0xFFFF0000u);
        pl[i >> 1] = pack_bf16x2(pv[0] - h0, pv[1] - h1);
      }
      l_run += psum;

      // ---- exchange P with the partner wave (same heads, other 32 slots) ----
      // The high parts go through s_p; the low parts through the RoPE chunk
      // columns 64..71 of the current tile, which PV does not read and every
      // wave has finished reading for QK (the s_max barrier above).
      uint8_t* s_plo = const_cast<uint8_t*>(tile) + 64 * 1024;
      *(u32x4*)(s_p + ((wave * 2 + 0) * 64 + lane) * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      *(u32x4*)(s_p + ((wave * 2 + 1) * 64 + lane) * 16) = u32x4{pk[4], pk[5], pk[6], pk[7]};
      *(u32x4*)(s_plo + ((wave * 2 + 0) * 64 + lane) * 16) = u32x4{pl[0], pl[1], pl[2], pl[3]};
      *(u32x4*)(s_plo + ((wave * 2 + 1) * 64 + lane) * 16) = u32x4{pl[4], pl[5], pl[6], pl[7]};
      lds_barrier();
      bf16x8 pf[4], pg[4];        // B operands per k-step: hi, lo
      {
        const u32x4 o0 = *(const u32x4*)(s_p + ((partner * 2 + 0) * 64 + lane) * 16);
        const u32x4 o1 = *(const u32x4*)(s_p + ((partner * 2 + 1) * 64 + lane) * 16);
        const u32x4 m0 = u32x4{pk[0], pk[1], pk[2], pk[3]};
        const u32x4 m1 = u32x4{pk[4], pk[5], pk[6], pk[7]};
        // k-step kst covers slots [16kst, 16kst+16), owned by wave half kst/2.
        pf[0] = __builtin_bit_cast(bf16x8, x == 0 ? m0 : o0);
        pf[1] = __builtin_bit_cast(bf16x8, x == 0 ? m1 : o1);
        pf[2] = __builtin_bit_cast(bf16x8, x == 1 ? m0 : o0);
        pf[3] = __builtin_bit_cast(bf16x8, x == 1 ? m1 : o1);
        const u32x4 q0 = *(const u32x4*)(s_plo + ((partner * 2 + 0) * 64 + lane) * 16);
        const u32x4 q1 = *(const u32x4*)(s_plo + ((partner * 2 + 1) * 64 + lane) * 16);
        const u32x4 n0 = u32x4{pl[0], pl[1], pl[2], pl[3]};
        const u32x4 n1 = u32x4{pl[4], pl[5], pl[6], pl[7]};
        pg[0] = __builtin_bit_cast(bf16x8, x == 0 ? n0 : q0);
        pg[1] = __builtin_bit_cast(bf16x8, x == 0 ? n1 : q1);
        pg[2] = __builtin_bit_cast(bf16x8, x == 1 ? n0 : q0);
        pg[3] = __builtin_bit_cast(bf16x8, x == 1 ? n1 : q1);
      }

      // ---- O^T += V^T . P^T over this wave's 256 columns ---------------------
      {
        const int i16 = lane & 15;
        const int nhalf = (lane >> 4) & 1;
        const int cb = 2 * nhalf + ((i16 & 3) >> 1);   // chunk & 3 of this lane's reads
        const int half8 = (i16 & 1) * 8;
        const uint8_t* vb0 = tile + (32 * x + cb) * 1024 + (((4 * g + (i16 >> 2)) ^ (4 * cb)) * 16) + half8;
        const uint8_t* vb1 = tile + (32 * x + cb) * 1024 + (((8 + 4 * g + (i16 >> 2)) ^ (4 * cb)) * 16) + half8;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
          for (int kst = 0; kst < 4; ++kst) {
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(vb0 + 4096 * ct + 256 * kst));
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(vb1 + 4096 * ct + 256 * kst));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kst], acc[ct], 0, 0, 0);
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pg[kst], acc[ct], 0, 0, 0);
          }
        }
      }

      vmask_cur = vmask_nxt;
      sc_cur = sc_nxt;
      idx_nxt = idx_after;
    }
  }

  // ---- epilogue: full denominator of this lane's head -----------------------
  const float l_wave = l_run + __shfl_xor(l_run, 32);
  if (lane < 32) s_l[x][hh] = l_wave;
  lds_barrier();
  const float l_head = s_l[0][hh] + s_l[1][hh];
  const bool any = l_head > 0.f;
  const float lse = any ? M_run + __builtin_amdgcn_logf(l_head) : kNegInf;
  float oscale = any ? 1.0f / l_head : 0.f;
  const bool head_ok = hh < a.h_q;

  if (!DIRECT) {
    const int64_t row = ((int64_t)job.s * a.s_q + t) * a.h_q + hh;
    if (head_ok) {
      float* orow = a.o_accum + row * 512;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = 256 * x + 32 * ct + 8 * q4 + 4 * g;
          f32x4 v = {acc[ct][4 * q4 + 0] * oscale, acc[ct][4 * q4 + 1] * oscale,
                     acc[ct][4 * q4 + 2] * oscale, acc[ct][4 * q4 + 3] * oscale};
          *(f32x4*)(orow + col) = v;
        }
      if (x == 0 && g == 0) a.lse_accum[row] = lse;
    }
  } else {
    if (a.sink != nullptr && any && head_ok) {
      const float z = a.sink[hh] * kLog2e - lse;
      oscale = oscale / (1.0f + __builtin_amdgcn_exp2f(z));
    }
    const int64_t row = (int64_t)t * a.h_q + hh;
    if (a.out_dtype == kOutFp8) {
      float amax = 0.f;
      if (head_ok)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[ct][i] * oscale));
      amax = warp_max(amax);
      if (lane == 0) s_red[wave] = amax;
      lds_barrier();
      amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      const float qscale = amax > 0.f ? amax / 448.0f : 1.0f;
      if (tid == 0) a.out_scale[t] = qscale;
      if (head_ok) {
        uint8_t* orow = (uint8_t*)a.out + row * 512;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int col = 256 * x + 32 * ct + 8 * q4 + 4 * g;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) w |= e4m3_encode((acc[ct][4 * q4 + e] * oscale) / qscale) << (8 * e);
            *(uint32_t*)(orow + col) = w;
          }
      }
    } else if (head_ok) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = 256 * x + 32 * ct + 8 * q4 + 4 * g;
          const float v0 = acc[ct][4 * q4 + 0] * oscale, v1 = acc[ct][4 * q4 + 1] * oscale;
          const float v2 = acc[ct][4 * q4 + 2] * oscale, v3 = acc[ct][4 * q4 + 3] * oscale;
          if (a.out_dtype == kOutF32) {
            *(f32x4*)((float*)a.out + row * 512 + col) = f32x4{v0, v1, v2, v3};
          } else {
            *(u32x2*)((uint16_t*)a.out + row * 512 + col) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          }
        }
    }
    if (a.lse_out != nullptr && head_ok && x == 0 && g == 0) a.lse_out[row] = lse;
  }
}

// ---------------------------------------------------------------------------
// Combine: O = sum_s 2^(LSE_s - M) O_s / sum_s 2^(LSE_s - M), then the sink and
// the cast.  bf16 / fp32 outputs: 128 threads per (token, head), 4 columns
// each.  FP8 output: one workgroup per token so the amax is a local reduction.
// ---------------------------------------------------------------------------
struct Merged {
  float lse, M, inv_w;
  bool any;
};

__device__ __forceinline__ Merged merge_weights(const CombineArgs& a, int t, int h) {
  const int64_t stride = (int64_t)a.s_q * a.h_q;
  const float* lp = a.lse_accum + (int64_t)t * a.h_q + h;
  float M = kNegInf;
  for (int s = 0; s < a.num_splits; ++s) M = fmaxf(M, lp[s * stride]);
  Merged m;
  m.M = M;
  m.any = M != kNegInf;
  float wsum = 0.f;
  if (m.any)
    for (int s = 0; s < a.num_splits; ++s) {
      const float ls = lp[s * stride];
      wsum += (ls == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ls - M);
    }
  m.lse = m.any ? M + __builtin_amdgcn_logf(wsum) : kNegInf;
  m.inv_w = m.any ? 1.0f / wsum : 0.f;
  return m;
}

__device__ __forceinline__ f32x4 merge_columns(const CombineArgs& a, const Merged& m, int t, int h, int col) {
  const int64_t stride = (int64_t)a.s_q * a.h_q;
  const float* lp = a.lse_accum + (int64_t)t * a.h_q + h;
  const float* op = a.o_accum + ((int64_t)t * a.h_q + h) * 512 + col;
  if (!m.any) return f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 o = {-0.f, -0.f, -0.f, -0.f};     // IEEE additive identity: keeps the sign of -0 terms
  for (int s = 0; s < a.num_splits; ++s) {
    const float ls = lp[s * stride];
    if (ls == kNegInf) continue;
    const float w = __builtin_amdgcn_exp2f(ls - m.M);
    const f32x4 v = *(const f32x4*)(op + s * stride * 512);
    o += w * v;
  }
  float f = m.inv_w;
  if (a.sink != nullptr) f = f / (1.0f + __builtin_amdgcn_exp2f(a.sink[h] * kLog2e - m.lse));
  return o * f;
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int hpb = 2;                               // heads per block
  const int blocks_per_token = (a.h_q + hpb - 1) / hpb;
  const int t = blockIdx.x / blocks_per_token;
  const int h = (blockIdx.x - t * blocks_per_token) * hpb + (threadIdx.x >> 7);
  if (h >= a.h_q) return;
  const int col = (threadIdx.x & 127) * 4;
  const Merged m = merge_weights(a, t, h);
  const f32x4 o = merge_columns(a, m, t, h, col);
  const int64_t row = (int64_t)t * a.h_q + h;
  if (a.out_dtype == kOutF32) {
    *(f32x4*)((float*)a.out + row * 512 + col) = o;
  } else {
    *(u32x2*)((uint16_t*)a.out + row * 512 + col) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  }
  if (a.lse_out != nullptr && (threadIdx.x & 127) == 0) a.lse_out[row] = m.lse;
}

// FP8 output: 1024 threads per token; 16 threads per head, 32 columns each.
__global__ __launch_bounds__(1024) void combine_fp8_kernel(CombineArgs a) {
  __shared__ float s_red[16];
  const int t = blockIdx.x;
  const int h = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const bool hv = h < a.h_q;
  f32x4 o[8];
  float amax = 0.f;
  Merged m = {kNegInf, kNegInf, 0.f, false};
  if (hv) {
    m = merge_weights(a, t, h);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[k] = merge_columns(a, m, t, h, (k * 16 + sub) * 4);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(o[k][0]), fabsf(o[k][1])), fmaxf(fabsf(o[k][2]), fabsf(o[k][3]))));
    }
  }
  amax = warp_max(amax);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) amax = fmaxf(amax, s_red[w]);
  const float qscale = amax > 0.f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) a.out_scale[t] = qscale;
  if (!hv) return;
  const int64_t row = (int64_t)t * a.h_q + h;
  uint8_t* orow = (uint8_t*)a.out + row * 512;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= e4m3_encode(o[k][e] / qscale) << (8 * e);
    *(uint32_t*)(orow + (k * 16 + sub) * 4) = w;
  }
  if (a.lse_out != nullptr && sub == 0) a.lse_out[row] = m.lse;
}

}  // namespace

hipError_t launch_decode_partial(const DecodeArgs& a, bool kv_fp8, hipStream_t stream) {
  const dim3 grid((unsigned)(a.s_q * a.num_splits));
  if (kv_fp8)
    hipLaunchKernelGGL((decode_kernel<true, false>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<false, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_direct(const DecodeArgs& a, bool kv_fp8, hipStream_t stream) {
  const dim3 grid((unsigned)a.s_q);
  if (kv_fp8)
    hipLaunchKernelGGL((decode_kernel<true, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<false, true>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.out_dtype == kOutFp8) {
    hipLaunchKernelGGL(combine_fp8_kernel, dim3((unsigned)a.s_q), dim3(1024), 0, stream, a);
  } else {
    const unsigned blocks = (unsigned)(a.s_q * ((a.h_q + 1) / 2));
    hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace smla
