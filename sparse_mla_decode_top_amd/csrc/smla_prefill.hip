// HIP kernels for split-KV FP8 prefill attention on MI355X (gfx950, CDNA4).
//
// The operation follows cudnn-frontend PR #768 ("split kv ports", commit
// messages and reviews): an FP8 SDPA prefill kernel with head dimension 128
// whose split form cuts each query tile's masked KV range into SPLIT_KV
// near-equal chunks of KV blocks (the remainder on the leading chunks; a chunk
// past the end is empty: O = 0, LSE = -inf), writes split-major partial O and
// LSE, and leaves the amax of the output to the combine, which owns the
// recombined O.  The sink counts once, in the combine (or in the direct
// epilogue when there is no split).
//
// prefill_kernel: one workgroup of 4 wave64s per (batch, 64-row query tile,
// HPW query heads of one KV head, split).  Wave w owns query rows
// [16w, 16w + 16) of the tile for each of its HPW heads: a K or V fragment read
// from LDS and converted to bf16 once feeds the matrix core HPW times (HPW = 2
// when a KV head serves an even number of query heads, measured 9% faster on
// the 4,096-token prompt than one head a workgroup; else 1).
//   * K and V blocks of 64 keys (e4m3, 8 KB each) are gathered with 16-byte
//     direct-to-LDS loads (global_load_lds_dwordx4) into kPStages stages:
//     while block b is computed, blocks b+1 .. b+kPStages-1 are in flight
//     (3 stages measured 9% faster than 4 on the 4,096-token prompt, whose 64 KB
//     of LDS allow one workgroup fewer a CU, and level with 2).
//     Keys past the batch's key count copy a zero row, so no padding row is
//     ever read.
//   * S^T[key][row] = K . Q^T on the bf16 matrix core: Q (once) and the K
//     fragments (8-byte LDS reads along a key row) are e4m3 codes converted to
//     bf16 in registers, exactly.  Each lane holds 16 scores of one query row.
//     The FP8 matrix core (v_mfma_f32_16x16x32_fp8_fp8) on the same codes was
//     measured on the MI355X at about 2e-5 relative error in a score (the LSE of
//     a row that sees one key is that key's score), twice the 1e-5 LSE bar; the
//     bf16 form measured 7e-7 on the same inputs.
//   * Softmax in log2 units against an integer frame M per row (the running
//     floor of the row maximum): the weight is p = 2^(t - M + 14), one fma and
//     one v_exp_f32, so p < 2^15.  A frame change rescales the accumulators by
//     an exact power of two.
//   * O^T[dim][row] += V^T . P^T on the f16 matrix core, P as one f16 term.
//     V^T fragments come from the 8-bit transposing LDS read ds_read_b64_tr_b8
//     of the e4m3 V tile, converted to f16 in registers (exact: every e4m3
//     value is an f16 value).  f16 keeps p to 2^-12 relative, which holds O
//     within about 1e-3 of the exact result for values of the inputs' size
//     (one bf16 term, 2^-9, does not: rows that see few keys reach 7e-3).  The
//     2^14 keeps every weight above 2^-28 of its row's largest out of f16's
//     subnormals, where the rounding would depend on the frame and so on the
//     split count.  The P^T fragment is the lane's own scores: its k-elements
//     are keys 4G .. 4G + 3 of one 16-key tile and 4G .. 4G + 3 of the next,
//     and the V^T reads fetch the same keys in the same order.
//   * Epilogue: O = acc * descale_v / l, LSE = (M - 14 + log2 l) * ln 2.  Split:
//     the partial and its LSE.  Direct: the sink, the cast, the LSE and the
//     amax (one atomic max per wave on the bits of |O|, a non-negative float).
//
// The workgroups that read the same K/V (one batch, split and KV head: every
// query tile and every query head of the head group) are numbered
// consecutively and placed on one XCD: block ids go to the 8 XCDs round robin,
// so logical workgroup (xcd * n + k) runs as block (k * 8 + xcd).
//
// prefill_combine_kernel: one wave per 4 consecutive (batch, row, head) rows
// in turn; a row's split LSEs come through scalar loads, and lane l merges
// dimensions 2l, 2l + 1 over the splits, applies the sink, casts, and the
// workgroup raises the amax once for its 64 rows.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "smla.h"
#include "smla_gfx950.h"
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kPRows = 64;              // query rows per tile: 4 waves x 16
constexpr int kPKeys = 64;              // keys per KV block
constexpr int kPDim = 128;              // head dimension (bytes per e4m3 row)
// Weights are taken as 2^(t - M + kPWeightShift): below 2^15 for f16, and
// out of its subnormals down to 2^-28 of the row's largest weight.
constexpr float kPWeightShift = 14.0f;
constexpr int kPTile = kPKeys * kPDim;  // bytes of one K or V block in LDS
constexpr float kPMasked = -3.0e38f;    // score of a masked key: its weight is exactly 0
constexpr float kPNoFrame = 3.0e38f;    // frame of a row that has not seen a key yet
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kPStages = 3;             // K/V blocks in LDS: one computed, up to two in flight (48 KB)
// Rows a combine wave merges in turn: the workgroups (16 waves) then raise the
// amax with 4x fewer atomics, which all land on one word (measured: with one
// row a wave the amax atomics cost about 4 us of the chunked prefill's combine).
constexpr int kPCombineRows = 4;

enum { kPOutBf16 = 0, kPOutF32 = 1 };

// Source of every key past the batch's key count.
__device__ __attribute__((aligned(256))) uint8_t g_zero_kv[kPDim];

// K / V block in LDS: key r is 128 bytes = 8 chunks of 16; chunk c sits at
// 16-byte position r * 8 + (c ^ kvsw(r)).  Both read streams -- 8-byte K reads
// of 16 keys x 2 chunks, and the V^T transpose reads of 32 keys x 1 chunk --
// then touch all 16 groups of four LDS banks twice: 2 cycles per 512 bytes.
__host__ __device__ constexpr int kvsw(int r) { return (r >> 1) & 7; }

struct PrefillWork {
  int b, s, hk, tile, h;      // h: the first of the workgroup's HPW query heads
};
// Logical workgroup id -> work item; the ones sharing a (batch, split, KV head)
// are consecutive.  A workgroup takes HPW consecutive query heads of one KV
// head's group.  Query tiles come last tile first: under the causal mask a
// tile's KV range grows with its index, and each XCD starts its workgroups in
// logical order, so the longest start first and the short ones fill in behind
// them (measured 15% faster on the 4,096-token prompt than first tile first).
template <int HPW>
__device__ __forceinline__ PrefillWork prefill_work(const PrefillArgs& a, int logical) {
  const int g = a.h_q / a.h_kv;
  PrefillWork w;
  int r = logical;
  const int hg = r % (g / HPW);
  r /= g / HPW;
  w.tile = a.n_tiles - 1 - r % a.n_tiles;
  r /= a.n_tiles;
  w.hk = r % a.h_kv;
  r /= a.h_kv;
  w.s = r % a.num_splits;
  w.b = r / a.num_splits;
  w.h = w.hk * g + hg * HPW;
  return w;
}

__device__ __forceinline__ int clamp_len(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// Waits for the oldest K/V block a wave gathers while the `ahead` younger ones
// stay in flight (4 direct-to-LDS loads a block and wave; vmcnt counts them in
// issue order).
template <int STAGES>
__device__ __forceinline__ void wait_block(int ahead) {
  static_assert(STAGES >= 2 && STAGES <= 4, "up to two blocks ahead");
  if (STAGES == 4 && ahead >= 2)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (STAGES >= 3 && ahead >= 1)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool CAUSAL, bool SPLIT, int STAGES, int HPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * 2 * kPTile];   // per stage: K, then V
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, G = lane >> 4;
  // The split form's combine owns the amax: it starts at 0 (the combine's
  // atomics come after this launch).
  if (SPLIT && a.amax_out != nullptr && blockIdx.x == 0 && tid == 0) *a.amax_out = 0.0f;
  const int per_xcd = (int)(gridDim.x >> 3);
  const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (logical >= a.n_work) return;                      // padding of the grid
  const PrefillWork w = prefill_work<HPW>(a, logical);
  const int sq = clamp_len(a.seqlen_q[w.b], a.sq_max);
  const int skv = clamp_len(a.seqlen_kv[w.b], a.skv_max);
  const int q0 = w.tile * kPRows;
  if (q0 >= sq) return;                                 // a tile past this batch's rows

  // The tile's masked KV range (the keys its last row may see) and this split's blocks of it.
  const int shift = skv - sq;
  const int last = min(sq, q0 + kPRows) - 1;
  const int kv_end = CAUSAL ? clamp_len(last + shift + 1, skv) : skv;
  const int n_blk = (kv_end + kPKeys - 1) / kPKeys;
  int b0 = 0, b1 = n_blk;
  if (SPLIT) {
    const int base = n_blk / a.num_splits, rem = n_blk - base * a.num_splits;
    b0 = w.s * base + min(w.s, rem);
    b1 = b0 + base + (w.s < rem ? 1 : 0);
  }

  const int i = q0 + 16 * wave + j;                     // this lane's query row
  const bool row_ok = i < sq;
  const int vis = CAUSAL ? clamp_len(i + shift + 1, skv) : skv;   // keys [0, vis) visible to row i
  // Keys every row of the wave sees (wave-uniform): blocks below it need no mask.
  const int vis_lo = CAUSAL ? clamp_len(q0 + 16 * wave + shift + 1, skv) : skv;

  float M[HPW], l_run[HPW];   // per head: integer frame of row i (log2 units), this lane's share of l
  f32x4 acc[HPW][8];          // O^T: dims 16 mt + 4G + e of row i, per head
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    M[hh] = kPNoFrame;
    l_run[hh] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[hh][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (b0 < b1) {
    // Q fragments (B operand of S^T = K . Q^T): row i, dims 32 ks + 8G .. +8,
    // converted to bf16 once (exact).
    bf16x8 qf[HPW][4];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const uint8_t* qrow =
          a.q + ((int64_t)(w.b * a.sq_max + min(i, sq - 1)) * a.h_q + w.h + hh) * kPDim + 8 * G;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[hh][ks] = e4m3x8_to_bf16(*(const u32x2*)(qrow + 32 * ks));
    }
    const uint32_t lds0 = lds_addr(smem);
    // Wave w gathers keys [16w, 16w + 16) of a block, K and V, in two groups of
    // 8 keys: lane l fetches chunk (l & 7) ^ kvsw(key) of key 8 grp + (l >> 3),
    // which lands in slot l & 7 of that key's row.
    auto gather = [&](int kb, int st) {
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        const int r = 16 * wave + 8 * grp + (lane >> 3);
        const int key = kb * kPKeys + r;
        const int c = (lane & 7) ^ kvsw(r);
        const int64_t off = ((int64_t)(w.b * a.skv_max + key) * a.h_kv + w.hk) * kPDim + c * 16;
        const bool ok = key < skv;
        const uint8_t* ks = ok ? a.k + off : g_zero_kv + c * 16;
        const uint8_t* vs = ok ? a.v + off : g_zero_kv + c * 16;
        const uint32_t lk = __builtin_amdgcn_readfirstlane(lds0 + st * 2 * kPTile + (16 * wave + 8 * grp) * kPDim);
        dma_one<0, 0, 0>(ks, lk);
        dma_one<0, 0, 0>(vs, lk + kPTile);
      }
    };
    // Per-lane LDS offsets of the operand reads.  K (k-step ks, key tile t):
    // key 16t + j, chunk 2 ks + (G >> 1), half G & 1.  V^T (k-step kk, dim
    // tile mt): lane j reads half j & 1 of key 32 kk + 16 (j >> 3) + 4G +
    // ((j >> 1) & 3), chunk mt.
    const int vr0 = 16 * (j >> 3) + 4 * G + ((j >> 1) & 3);
    // V^T read offsets of the 16 (k-step, dim tile) fragments, one register each
    // (opaque, so that the compiler keeps them whole instead of re-adding a row
    // and a chunk part at every read); the stage goes in as an immediate.
    uint32_t voff[2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        voff[kk][mt] = opaque((32 * kk + vr0) * kPDim + (j & 1) * 8 + ((mt ^ kvsw(32 * kk + vr0)) * 16));

    // Blocks b0 .. b0 + STAGES - 2 go out first; each iteration then waits for
    // its own block only and refills the stage the previous block used.
#pragma unroll
    for (int pb = 0; pb < STAGES - 1; ++pb)
      if (b0 + pb < b1) gather(b0 + pb, pb);
    // One block of keys.  Its stage is a compile-time constant (the loop below is
    // unrolled over the stages), so every LDS operand address is a loop-invariant
    // lane offset plus an instruction immediate, with no add of a stage base.
    auto block = [&](const int kb, auto stage) __attribute__((always_inline)) {
      constexpr int st = decltype(stage)::value;
      wait_block<STAGES>(min(STAGES - 2, b1 - 1 - kb));   // this wave's share of block kb has landed
      lds_barrier();            // ... and every wave's; block kb - 1 fully read
      if (kb + STAGES - 1 < b1) gather(kb + STAGES - 1, (st + STAGES - 1) % STAGES);
      const uint32_t kt = lds0 + st * 2 * kPTile, vt = kt + kPTile;

      // ---- S^T = K . Q^T: four key tiles of 16, four k-steps of 32 dims; one
      // converted K fragment feeds every head of the wave
      f32x4 sacc[HPW][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) sacc[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int r = 16 * t + j;
          const uint32_t addr = kt + r * kPDim + (((2 * ks + (G >> 1)) ^ kvsw(r)) * 16) + (G & 1) * 8;
          const bf16x8 kf = e4m3x8_to_bf16(*(const __attribute__((address_space(3))) u32x2*)(uintptr_t)addr);
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh)
            sacc[hh][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[hh][ks], sacc[hh][t], 0, 0, 0);
        }
      }

      // ---- softmax per head: lane scores of row i, keys kb*64 + 16t + 4G + e
      const bool full = kb * kPKeys + kPKeys <= vis_lo;   // every key of the block visible to every row (uniform)
      f16x8 ph[HPW][2];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        // The row maximum is taken on the raw scores: the scale is positive (the
        // host rejects any other), so the largest scaled score is the scale times
        // the largest raw one, and each weight takes one fma for its exponent.
        // (The empty volatile statements keep the branches as uniform jumps: the
        // compiler would otherwise evaluate both sides and select.)
        const float c = a.scale_log2;
        float sv[16];
        if (full) {
          asm volatile("");
#pragma unroll
          for (int k = 0; k < 16; ++k) sv[k] = sacc[hh][k >> 2][k & 3];
        } else {
          asm volatile("");
          // key kb*64 + 16(k >> 2) + 4G + (k & 3) is visible iff its offset in the
          // lane's keys, 16(k >> 2) + (k & 3), is below lim: compares with constants
          const int lim = vis - kb * kPKeys - 4 * G;
#pragma unroll
          for (int k = 0; k < 16; ++k) sv[k] = 16 * (k >> 2) + (k & 3) < lim ? sacc[hh][k >> 2][k & 3] : kPMasked;
        }
        float mr = kPMasked;
#pragma unroll
        for (int k = 0; k < 16; ++k) mr = fmaxf(mr, sv[k]);
        mr = rows_max(mr);                               // the four lanes of row i
        const bool any = mr > kPMasked;
        const float fm = floorf(mr * c);
        const float M_new = !any ? M[hh] : (M[hh] == kPNoFrame ? fm : fmaxf(M[hh], fm));
        const bool moved = any && M[hh] != kPNoFrame && M_new != M[hh];
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {   // a row took a new frame: rescale by an exact power of two
          asm volatile("");
          const float f =
              moved ? __builtin_amdgcn_ldexpf(1.0f, (int)__builtin_amdgcn_fmed3f(M[hh] - M_new, -256.f, 0.f)) : 1.0f;
          l_run[hh] *= f;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) acc[hh][mt] = acc[hh][mt] * f;
        }
        M[hh] = M_new;
        // p = 2^(s c - M + kPWeightShift) < 2^15.  A masked key (s = -3e38) gets
        // p = 0, since the host keeps the scale at 2^-100 or more, and so does
        // every key of a row with no frame yet (M = 3e38).
        const float nM = kPWeightShift - M_new;
        float pv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sv[k], c, nM));
          l_run[hh] += p;
          pv[k] = p;
        }
        // P^T fragments of k-step kk: keys 4G .. +3 of tiles 2kk and 2kk + 1, in f16
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 h4;
#pragma unroll
          for (int q = 0; q < 4; ++q) h4[q] = pack_f16x2(pv[8 * kk + 2 * q], pv[8 * kk + 2 * q + 1]);
          ph[hh][kk] = __builtin_bit_cast(f16x8, h4);
        }
      }

      // ---- O^T += V^T . P^T: eight dim tiles of 16, two k-steps of 32 keys; one
      // converted V^T fragment feeds every head of the wave
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          typedef int i32x2v __attribute__((ext_vector_type(2)));
          const uint32_t addr = vt + voff[kk][mt];
          const i32x2v r =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2v*)(uintptr_t)addr);
          const f16x8 vf = e4m3x8_to_f16(u32x2{(uint32_t)r[0], (uint32_t)r[1]});
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh)
            acc[hh][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph[hh][kk], acc[hh][mt], 0, 0, 0);
        }
      }
    };
    for (int kb = b0; kb < b1; kb += STAGES) {
      block(kb, std::integral_constant<int, 0>{});
      if (kb + 1 < b1) block(kb + 1, std::integral_constant<int, 1 % STAGES>{});
      if (STAGES > 2 && kb + 2 < b1) block(kb + 2, std::integral_constant<int, 2 % STAGES>{});
      if (STAGES > 3 && kb + 3 < b1) block(kb + 3, std::integral_constant<int, 3 % STAGES>{});
    }
  }

  // ---- epilogue per head: row i's denominator over its four lanes; O = acc * descale_v / l
  float amax = 0.f;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = w.h + hh;
    const float l = rows_sum(l_run[hh]);
    const bool has = l > 0.f;
    const float lse = has ? (M[hh] - kPWeightShift + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
    float oscale = has ? a.descale_v / l : 0.f;
    if (!SPLIT && a.sink != nullptr && has)
      oscale = oscale / (1.0f + __builtin_amdgcn_exp2f((a.sink[h] - lse) * kLog2e));
    if (row_ok) {
      const int64_t row = (int64_t)(w.b * a.sq_max + i) * a.h_q + h;
      if (SPLIT) {
        const int64_t prow = (int64_t)w.s * a.batch * a.sq_max * a.h_q + row;
        float* dst = a.o_part + prow * kPDim + 4 * G;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) *(f32x4*)(dst + 16 * mt) = acc[hh][mt] * oscale;
        if (G == 0) a.lse_part[prow] = lse;
      } else {
        if (a.out_dtype == kPOutF32) {
          float* dst = (float*)a.out + row * kPDim + 4 * G;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const f32x4 o = acc[hh][mt] * oscale;
            *(f32x4*)(dst + 16 * mt) = o;
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3]))));
          }
        } else {
          uint16_t* dst = (uint16_t*)a.out + row * kPDim + 4 * G;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const f32x4 o = acc[hh][mt] * oscale;
            *(u32x2*)(dst + 16 * mt) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3]))));
          }
        }
        if (G == 0 && a.lse_out != nullptr) a.lse_out[row] = lse;
      }
    }
  }
  if (!SPLIT && a.amax_out != nullptr) {
    amax = wave_max(amax);
    if (lane == 0)
      __hip_atomic_fetch_max((uint32_t*)a.amax_out, __float_as_uint(amax), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The direct form's amax starts at 0 before the attention kernel's atomics.
__global__ void prefill_amax_init_kernel(float* amax_out) { *amax_out = 0.0f; }

// One wave per (batch, row, head) row r = 16 * block + wave; lane l merges
// dims 2l, 2l + 1.  Lane s holds split s's LSE; the partial pieces of the
// first 8 splits are requested before the weights are known.  The workgroup's
// amax meets in LDS and raises amax_out once, and only when it is larger than
// the value already there.
__global__ __launch_bounds__(1024) void prefill_combine_kernel(PrefillArgs a) {
  __shared__ float s_amax[16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.batch * a.sq_max * a.h_q;      // one split's rows
  const int S = a.num_splits;
  float amax = 0.f;
  for (int k = 0; k < kPCombineRows; ++k) {
    const int64_t r = ((int64_t)blockIdx.x * 16 + wave) * kPCombineRows + k;    // this wave's row (uniform)
    bool live = r < rows;
    int h = 0;
    if (live) {
      h = (int)(r % a.h_q);
      const int64_t bi = r / a.h_q;
      const int i = (int)(bi % a.sq_max);
      const int b = (int)(bi / a.sq_max);
      live = i < clamp_len(a.seqlen_q[b], a.sq_max);               // not a padding row
    }
    if (live) {
      // The row's split LSEs are the same for every lane: scalar loads (the
      // partials are only read here).
      typedef const __attribute__((address_space(4))) float* clse_t;
      const clse_t lse = (clse_t)(const void*)a.lse_part;
      float M = kNegInf;
      for (int s = 0; s < S; ++s) M = fmaxf(M, lse[(int64_t)s * rows + r]);
      const float* op = a.o_part + r * kPDim + 2 * lane;
      f32x2 o = {0.f, 0.f};
      float wsum = 0.f;
      for (int s0 = 0; s0 < S; s0 += 8) {
        f32x2 x[8];
        float w[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (s0 + c < S) {
            x[c] = *(const f32x2*)(op + (int64_t)(s0 + c) * rows * kPDim);
            const float ls = lse[(int64_t)(s0 + c) * rows + r];
            w[c] = (M == kNegInf || ls == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((ls - M) * kLog2e);
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (s0 + c < S) {
            o = o + w[c] * x[c];
            wsum += w[c];
          }
        }
      }
      const bool none = M == kNegInf;
      const float lse_r = none ? kNegInf : M + __builtin_amdgcn_logf(wsum) * kLn2;
      float f = none ? 0.f : 1.0f / wsum;
      if (a.sink != nullptr && !none) f = f / (1.0f + __builtin_amdgcn_exp2f((a.sink[h] - lse_r) * kLog2e));
      o = o * f;
      if (a.out_dtype == kPOutF32)
        *(f32x2*)((float*)a.out + r * kPDim + 2 * lane) = o;
      else
        *(uint32_t*)((uint16_t*)a.out + r * kPDim + 2 * lane) = pack_bf16x2(o[0], o[1]);
      if (lane == 0 && a.lse_out != nullptr) a.lse_out[r] = lse_r;
      amax = fmaxf(amax, fmaxf(fabsf(o[0]), fabsf(o[1])));
    }
  }
  if (a.amax_out == nullptr) return;
  amax = wave_max(amax);
  if (lane == 0) s_amax[wave] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) v = fmaxf(v, s_amax[k]);
    uint32_t* am = (uint32_t*)a.amax_out;
    if (__float_as_uint(v) > __hip_atomic_load(am, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      __hip_atomic_fetch_max(am, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool split, hipStream_t stream) {
  if (!split && a.amax_out != nullptr) hipLaunchKernelGGL(prefill_amax_init_kernel, dim3(1), dim3(1), 0, stream, a.amax_out);
  // Two query heads a workgroup when a KV head has an even number of them.
  const bool pair = (a.h_q / a.h_kv) % 2 == 0;
  const int n_work = pair ? a.n_work / 2 : a.n_work;
  PrefillArgs b = a;
  b.n_work = n_work;
  const dim3 grid((unsigned)((n_work + 7) / 8 * 8));
#define SMLA_PREFILL(C, S, H) hipLaunchKernelGGL((prefill_kernel<C, S, kPStages, H>), grid, dim3(256), 0, stream, b)
  if (pair) {
    if (a.causal && split) SMLA_PREFILL(true, true, 2);
    else if (a.causal) SMLA_PREFILL(true, false, 2);
    else if (split) SMLA_PREFILL(false, true, 2);
    else SMLA_PREFILL(false, false, 2);
  } else {
    if (a.causal && split) SMLA_PREFILL(true, true, 1);
    else if (a.causal) SMLA_PREFILL(true, false, 1);
    else if (split) SMLA_PREFILL(false, true, 1);
    else SMLA_PREFILL(false, false, 1);
  }
#undef SMLA_PREFILL
  return hipGetLastError();
}

hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.sq_max * a.h_q;
  const int64_t per_wg = 16 * kPCombineRows;
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((rows + per_wg - 1) / per_wg)), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
