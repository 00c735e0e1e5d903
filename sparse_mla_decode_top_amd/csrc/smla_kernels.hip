// HIP kernels for split-KV sparse MLA decode on MI355X (gfx950, CDNA4).
//
// The operation follows FlashMLA PR #25 ("What changes": (query token, KV
// split) jobs, each walking its own block range and writing an fp32 partial
// normalised by its own denominator plus a log2-space LSE), "The Split-K
// Dispatch" ("The LSE Combine Strategy": merge with exp2 weights relative to
// the largest LSE) and cudnn-frontend PR #768 (near-equal block ranges with
// the remainder on the leading splits; an empty split is O = 0, LSE = -inf).
//
// Kernels, by launch (CS = workgroups a job takes):
//   * decode_kernel8p (CS = 1: 64 heads, or a direct FP8 output, whose scale
//     needs every head and column of a token; fewer heads are then padded to
//     64): 8 waves, all heads and columns.
//   * decode_kernel8h (64 heads, CS = 2): 8 waves, half of the heads each.
//   * decode_kernel4t (CS = h_q / 16 head tiles x 1, 2 or 4 column parts): 4
//     waves, one 16-head tile each (and a half or a quarter of its columns).
//     The head-part kernels repeat a head tile's QK^T only across its column
//     parts.
//   * decode_kernel8m: a mixed launch for more jobs than compute units
//     (decode_kernel8p's body, then decode_kernel8h's for a short last round).
// What they share:
//   * The 64 slots of a KV block share one LDS tile, gathered by index with
//     16-byte direct-to-LDS loads (global_load_lds_dwordx4) in which 8 lanes
//     fetch one contiguous 128-byte segment of a row (FP8 pool: 4 lanes a
//     64-byte segment of e4m3 codes, converted to bf16 in registers as the
//     MFMA operands are read); two tiles double-buffer the gather of block
//     b+1 behind the compute of block b, its DMAs spread over block b's QK^T
//     MFMAs.  Masked slots are never read: their tile rows are copied from a
//     zero row.
//   * S^T[slot][head] = K . Q^T and O^T[col][head] = V^T . P^T use
//     v_mfma_f32_16x16x32_bf16; every lane holds one head's scores and
//     accumulators.  Q is staged through LDS and kept in VGPRs (72 per lane);
//     V^T is read from the row-major tile with the gfx950 transpose load
//     ds_read_b64_tr_b16.
//   * The waves that share a head tile score a part of each block's slots
//     each, trade their bf16 weights through LDS and accumulate every slot
//     into their own part of the columns; the two waves of a SIMD in the
//     8-wave kernels score different slots, so the hardware overlaps one's
//     softmax and LDS reads with the other's MFMAs.
//   * Softmax in log2 units against an integer frame M per head, shared by
//     the waves of the head: each weight is p = 2^(t - M), one v_exp_f32.  M
//     is the floor of the head's first non-empty block maximum and never
//     moves inside a pass, so the accumulators are touched by MFMAs only.  A
//     later score above M + 64 would risk overflow: the job then runs once
//     more with M = floor of the largest score seen, which bounds every p by
//     2.  The denominator sums the unrounded fp32 weights.
//   * P enters the PV product as two bf16 terms, hi = bf16(p) and
//     lo = bf16(p - hi), sharing each V^T operand: a bf16-rounded P alone
//     leaves O errors near 4e-3 when a few slots dominate (one 64-slot block);
//     hi + lo carries p to about 2^-17 relative.
//   * Outputs are staged through LDS and stored in whole-line pieces.
//   * With more jobs than compute units, a last round that fills at most half
//     of them takes 2, 4 or 8 parts (64 heads: 2, in the same launch,
//     decode_kernel8m).
//
// combine kernel: split-major partials -> final output (+ sink, cast).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "smla.h"
#include "smla_gfx950.h"
#include "smla_internal.h"

// Split partials of sparse_mla_decode_noalloc: one copy on every GPU the
// library runs on.  In host code `scratch` names a host-side stand-in, never
// the device memory: only the address hipGetSymbolAddress returns for the
// current device (noalloc_scratch below) is handed to kernels.
static __device__ __align__(256) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace smla {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 64;                         // slots per KV block
constexpr int kTileBytes = kBlk * 1152;          // 64 bf16 rows of 576
constexpr int kCodeTileBytes = kBlk * 576;       // 64 e4m3 rows of 576
constexpr int kQOffset = kTileBytes;             // LDS byte offset of the staged Q rows
constexpr float kFrameSlack = 64.0f;     // scores may exceed a head's frame M by this much
// Score of a masked slot: finite and below any real score; its weight
// 2^(t - M) is exactly 0 for every frame.
constexpr float kMaskedScore = -3.0e38f;
// Frame of a head that has not seen a valid slot yet: every weight is then 0.
constexpr float kNoFrame = 3.0e38f;

enum OutDtype { kOutBf16 = 0, kOutF32 = 1, kOutFp8 = 2 };

// Zeros: a pool row that the spread-out gather copies for masked slots, so
// each of its DMA instructions is issued by every lane, branch free (its first
// 1152 bytes), and an fp32 partial row that the combine loads for the split
// slots of a chunk past the split count (all 2048).
__device__ __attribute__((aligned(256))) uint8_t g_zero_row[2048];

// ---------------------------------------------------------------------------
// LDS tile layout ("octet-major").  A bf16 row is 72 chunks of 16 bytes (8
// elements), grouped in 9 octets of 8 chunks (128 bytes).  Chunk c of tile row
// r sits at 16-byte position
//     (c >> 3) * 512 + r * 8 + ((c & 7) ^ (r & 7)).
// * Gather: one load instruction fills one octet of 8 rows; lanes 8k..8k+7
//   fetch the 128 contiguous bytes of one row (in swizzled order).
// * The XOR of the chunk slot with the low row bits makes both operand read
//   streams bank-conflict free on the gfx950 LDS (64 banks, 256 B/clk): the
//   QK^T reads (16 B per lane, 16 rows x 4 chunks per instruction) and the PV
//   transpose reads (8 B per lane, 16 rows x 2 chunks).  This was measured
//   with the LDS bank-conflict counter over the kernel's exact address
//   streams; several XOR patterns that look conflict free on paper are 2-way
//   conflicted there.
// The FP8 code tile has a layout of its own (below).
// ---------------------------------------------------------------------------
// Chunk-slot XOR of tile row r.
__host__ __device__ constexpr int rsw(int r) { return r & 7; }


// ---------------------------------------------------------------------------
// FP8 code tile (e4m3 pool rows), "quartet-major" and swizzled.  A row is 36
// chunks of 16 codes, grouped in 9 quartets of 4 chunks (64 bytes).  Chunk c
// of tile row r sits at 16-byte position
//     (c >> 2) * 256 + r * 4 + ((c & 3) ^ csw(r)),   csw(r) = (r >> 2) & 3.
// * Gather: one load instruction fills one quartet of 16 rows; lanes 4k..4k+3
//   fetch the 64 contiguous bytes of one row, in swizzled order.
// * The MFMA operands are read from the codes and converted to bf16 in
//   registers (exact): K fragments as 8-byte reads along a row, V^T fragments
//   with the gfx950 8-bit transpose read ds_read_b64_tr_b8.  In each group of
//   16 lanes that read reads 8 bytes per lane and hands lane i, as its byte k,
//   byte (i & 7) of what lane 2k + (i >> 3) read (measured on the MI355X): with
//   lane j pointed at half (j & 1) of row R(j >> 1), lane i receives column i
//   of rows R(0) .. R(7) -- 8 slots of one value column, the V^T operand.
//   The XOR puts both read streams on distinct LDS banks (2 cycles per
//   512-byte read).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int csw(int r) { return (r >> 2) & 3; }

// Byte offset within a quartet of the chunk that gathering lane l fetches: row
// l >> 2 of a group of 16 rows starting at a multiple of 16.
__device__ __forceinline__ int fp8_gather_chunk(int lane) { return ((lane & 3) ^ csw(lane >> 2)) * 16; }

// Per-lane byte offsets of the FP8 operand reads (lane = 16 G + j).
//   k[p]: K fragment of a k-step of parity p, row j of the slot tile (add
//         1024 per slot tile and 4096 per k-step pair): dims 32 ks + 8G .. +8,
//         i.e. chunk 2 p + (G >> 1), half G & 1.
//   v[m]: V^T fragment of a column chunk c with c & 3 = m (add 4096 per
//         quartet c >> 2 and 2048 per 32-slot k-step).  Its k-elements are
//         the slots that the weight operand holds, as in the bf16 fragment:
//         4G .. 4G + 3, then 16 + 4G .. 16 + 4G + 3 of the k-step; so lane j
//         reads half j & 1 of slot 16 (j >> 3) + 4G + ((j >> 1) & 3), whose
//         csw is G.
struct Fp8Offsets {
  int k[2];
  int v[4];
};
__device__ __forceinline__ Fp8Offsets fp8_offsets(int lane) {
  const int j = lane & 15, G = lane >> 4;
  Fp8Offsets o;
#pragma unroll
  for (int p = 0; p < 2; ++p) o.k[p] = j * 64 + (((2 * p + (G >> 1)) ^ csw(j)) * 16) + (G & 1) * 8;
  const int vrow = (16 * (j >> 3) + 4 * G + ((j >> 1) & 3)) * 64 + (j & 1) * 8;
#pragma unroll
  for (int m = 0; m < 4; ++m) o.v[m] = vrow + ((m ^ G) * 16);
  return o;
}
__device__ __forceinline__ bf16x8 fp8_kfrag(uint32_t addr) {
  return e4m3x8_to_bf16(*(const __attribute__((address_space(3))) u32x2*)(uintptr_t)addr);
}
__device__ __forceinline__ bf16x8 fp8_vfrag(uint32_t addr) {
  typedef int i32x2v __attribute__((ext_vector_type(2)));
  const i32x2v r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2v*)(uintptr_t)addr);
  return e4m3x8_to_bf16(u32x2{(uint32_t)r[0], (uint32_t)r[1]});
}

// Nine 16-byte direct-to-LDS loads from one row per lane.  The hardware adds
// the instruction offset to BOTH addresses (LDS address = m0 + offset +
// 16*lane), so m0 advances by (LDS step - global step).  Issued as one inline
// assembly block so that the compiler neither touches m0 in between nor
// inserts a vmcnt wait in front of the LDS reads of the other tile buffer (it
// cannot tell the prefetch buffer from the one being read); the kernel waits
// explicitly.  m0 is saved and restored; one wait state follows each m0 write.
#define SMLA_DMA_OP(OPND, M0STEP, OFF) \
  "s_add_u32 m0, m0, " #M0STEP "\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %" #OPND ", off offset:" #OFF "\n\t"
#define SMLA_DMA(M0STEP, OFF) SMLA_DMA_OP(1, M0STEP, OFF)
// bf16 tile: octet o of a row -> global +128o, LDS +8192o  (m0 step 8064)
__device__ __forceinline__ void dma_octets(const void* gptr, uint32_t lds_base_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      SMLA_DMA(8064, 128) SMLA_DMA(8064, 256) SMLA_DMA(8064, 384) SMLA_DMA(8064, 512)
      SMLA_DMA(8064, 640) SMLA_DMA(8064, 768) SMLA_DMA(8064, 896) SMLA_DMA(8064, 1024)
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base_uniform)
      : "memory");
}
// FP8 code tile: quartet q of a row -> global +64q, LDS +4096q  (m0 step 4032)
__device__ __forceinline__ void dma_quartets(const void* gptr, uint32_t lds_base_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      SMLA_DMA(4032, 64) SMLA_DMA(4032, 128) SMLA_DMA(4032, 192) SMLA_DMA(4032, 256)
      SMLA_DMA(4032, 320) SMLA_DMA(4032, 384) SMLA_DMA(4032, 448) SMLA_DMA(4032, 512)
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base_uniform)
      : "memory");
}
// First index of a job and its Q rows in one block: the index load is issued,
// then the 9 DMAs of this wave's 8 Q rows (as a KV gather), and only the index
// is waited for (vmcnt counts completions in issue order, so the 9 DMAs stay
// in flight).  One asm statement, so that the compiler neither reads the index
// register before it has landed nor adds a wait of its own that would cover
// the DMAs.
__device__ __forceinline__ int load_idx_and_q1(const int32_t* idx_ptr, const void* q0, uint32_t lds0_uniform) {
  int idx;
  uint32_t saved;
  asm volatile(
      "global_load_dword %0, %2, off\n\t"
      "s_mov_b32 %1, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      SMLA_DMA_OP(3, 8064, 128) SMLA_DMA_OP(3, 8064, 256) SMLA_DMA_OP(3, 8064, 384) SMLA_DMA_OP(3, 8064, 512)
      SMLA_DMA_OP(3, 8064, 640) SMLA_DMA_OP(3, 8064, 768) SMLA_DMA_OP(3, 8064, 896) SMLA_DMA_OP(3, 8064, 1024)
      "s_nop 0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_waitcnt vmcnt(9)"
      : "=&v"(idx), "=&s"(saved)
      : "v"(idx_ptr), "v"(q0), "s"(lds0_uniform)
      : "memory");
  return idx;
}
#undef SMLA_DMA
#undef SMLA_DMA_OP


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

// FP8 output through the combine (see the combine kernels below).  The two
// counter words of token t: [0] workgroups counted in, [1] the bits
// of the largest |O| seen (a non-negative float).
__device__ __forceinline__ uint32_t* fp8_sync_words(void* out, int t, int h_q) {
  return (uint32_t*)((uint8_t*)out + (int64_t)t * h_q * 512);
}

// Seeds token t's FP8 combine (one thread per token).
__device__ __forceinline__ void seed_fp8_combine(float* out_scale, void* out, int t, int h_q) {
  out_scale[t] = -0.0f;
  *(u32x2*)fp8_sync_words(out, t, h_q) = u32x2{0u, 0u};
}

// Job decode shared by every wave.  Job id = token * num_splits + split; a
// launch covers the jobs from job0 on.  With 2^lg_parts > 1 parts a job, the
// workgroups of a job are 8 block ids apart in groups of 8 * 2^lg_parts (blocks
// are spread over the 8 XCDs round robin, so all of them land on one XCD and
// share its L2 for the job's rows).  Blocks [b0, b1) of split s: near-equal
// ranges, the remainder on the leading splits, empty past the end.  part:
// which share of the job's heads and output columns this workgroup owns.
struct Job {
  int t, s, b0, b1, part;
  bool live;
};
__device__ __forceinline__ Job decode_job(int block, int lg_parts, int num_splits, int n_blocks, int job0,
                                          int n_jobs) {
  Job j;
  int id = block;
  j.part = (id >> 3) & ((1 << lg_parts) - 1);
  id = ((id >> 3) >> lg_parts) * 8 + (id & 7);
  id += job0;
  j.live = id < n_jobs;
  j.t = id / num_splits;
  j.s = id - j.t * num_splits;
  const int base = n_blocks / num_splits, rem = n_blocks - base * num_splits;
  j.b0 = j.s * base + min(j.s, rem);
  j.b1 = j.b0 + base + (j.s < rem ? 1 : 0);
  return j;
}

// A job's index list: lane l holds slot l of a 64-slot block.  The load
// address is clamped into the token's list so that it is issued
// unconditionally (no divergent branch, hence no early wait on it); slots past
// the split or the list are masked where the index is used, and so is an
// index outside the pool.
struct JobIndices {
  const int32_t* row;                 // the token's top-k list
  int topk, b1;                       // list length; end of the job's block range
  int64_t n_pool;
  __device__ __forceinline__ int load(int b, int lane) const { return row[min(b * kBlk + lane, topk - 1)]; }
  __device__ __forceinline__ bool slot_in(int b, int lane) const { return b < b1 && b * kBlk + lane < topk; }
  __device__ __forceinline__ bool valid(int idx) const { return idx >= 0 && (int64_t)idx < n_pool; }
};

// The global address a lane's gather DMAs start from: its piece of pool row
// `row_idx`, or of the zero row when the row is masked.  bf16: 8 lanes a row,
// chunk (l & 7) ^ (row & 7) of each 128-byte octet; FP8 codes: 4 lanes a row,
// the quartet chunk of fp8_gather_chunk.
template <bool KV_FP8>
__device__ __forceinline__ const uint8_t* gather_src(const DecodeArgs& a, int row_idx, bool valid, int lane) {
  return (valid ? a.kv + (int64_t)row_idx * a.row_stride_bytes : g_zero_row) +
         (KV_FP8 ? fp8_gather_chunk(lane) : (((lane & 7) ^ rsw(lane >> 3)) * 16));
}

// The first block's wait for this wave's Q rows, which were issued first:
// vector memory operations complete in issue order, so the block's DMAS
// gather DMAs and, with the look-ahead, the next index load stay in flight.
template <bool PREFETCH, int DMAS>
__device__ __forceinline__ void wait_q_rows() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMAS + (PREFETCH ? 1 : 0)) : "memory");
}

// A head tile's 18 Q fragments (B operand of S^T = K . Q^T: head, dims
// 32 ks + 8 G .. +8) from the staged Q rows at LDS address qt, kb0 / kb1 being
// the lane's offsets for even / odd k-steps.
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[18], uint32_t qt, int kb0, int kb1) {
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    const uint32_t qp = qt + ((ks & 1) ? kb1 : kb0) + (ks >> 1) * 8192;
    qf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)qp;
  }
}

// One block's gather in the 8-wave kernels, the lane's source from gather_src.
// bf16: wave w fills rows [8w, 8w + 8) of the tile; FP8: waves 0-3 fill rows
// [16w, 16w + 16) of the code tile.  9 DMAs a gathering wave.
template <bool KV_FP8>
__device__ __forceinline__ void gather_block8(const uint8_t* src, uint32_t tile_lds0, int buf, int wave) {
  if (!KV_FP8)
    dma_octets(src, __builtin_amdgcn_readfirstlane(tile_lds0 + buf * kTileBytes + wave * 1024));
  else if (wave < 4)
    dma_quartets(src, __builtin_amdgcn_readfirstlane(tile_lds0 + buf * kCodeTileBytes + wave * 1024));
}

// End of a pass, in every wave of the workgroup: posts the wave's largest
// score, its denominator (the row sum of l_run, which l_run becomes) and its
// overflow flag in its weight-exchange slot (floats [0, 16), [16, 32), int 32)
// and returns whether any of the NW waves overflowed.  The two barriers order
// the posts after every wave's last reads of the tiles and the weights, and
// before the reads of the other waves' posts.
template <int NW>
__device__ __forceinline__ bool post_pass(bool overflow, float m_seen, float& l_run, float* pex_own,
                                          const uint8_t* pex0, int slot_bytes, int hl, int G, int lane) {
  const float l_w = rows_sum(l_run);
  const bool ov = __any(overflow);
  lds_barrier();
  if (G == 0) {
    pex_own[hl] = m_seen;
    pex_own[16 + hl] = l_w;
  }
  if (lane == 0) ((int*)pex_own)[32] = ov ? 1 : 0;
  lds_barrier();
  l_run = l_w;
  int any_ov = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) any_ov |= ((const int*)(pex0 + v * slot_bytes))[32];
  return any_ov != 0;
}

// ---------------------------------------------------------------------------
// The attention kernels' template flags.  KV_FP8: pool rows are e4m3 codes +
// a row scale.  DIRECT: single-split job writing the final output (sink +
// cast fused).  PREFETCH: some job has more than one block, so each block
// gathers the next one (for a job's last block the gather copies the zero row
// into the idle buffer, keeping the loop free of branches).  The fields that
// the first instructions need come as leading scalar arguments, which the
// build asks to be preloaded into SGPRs at wave launch: the index and Q loads
// then issue without waiting for a kernel-argument load.
// ---------------------------------------------------------------------------

// The 8-wave kernels below (two waves per SIMD): 64 heads, 512 threads.
constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;

// ---------------------------------------------------------------------------
// decode_kernel8p: one 8-wave workgroup per job that owns all 512 output
// columns (64 heads, either pool), for launches with a single column part.
// The two waves on a SIMD own the same 16 heads and each scores one 32-slot
// half of every block.  Here they trade their bf16
// weights through LDS, and each wave accumulates every slot of the block into
// its own half of the columns (256): 64 accumulator registers a wave, which
// keeps two waves per SIMD without a second workgroup repeating QK^T.  The
// two halves of a head share one integer frame, agreed on in the first block
// that has a valid slot, so their weights add into one accumulator.
// LDS: the two tiles and the weight exchange fill the 160 KB exactly; the
// frame, end-of-pass and denominator exchanges reuse the weight area, and
// validity comes from a ballot of the block's indices.  KV_FP8: the two code
// tiles take the first bf16 tile's space, waves 0-3 gather them (as
// decode8h_body), the Q rows are staged over the second code tile (free until
// the first block's look-ahead gather, which follows a barrier) and the
// block's row scales follow the Q rows.
// ---------------------------------------------------------------------------
// LDS of decode_kernel8p: the two tiles, then the weight exchange.
constexpr int kLds8pBytes = 2 * kTileBytes + kWaves8 * 2048;
constexpr int kLds8pQFp8 = kCodeTileBytes;                   // FP8: the staged Q rows
constexpr int kLds8pScaleFp8 = kCodeTileBytes + kTileBytes;  // FP8: [2][kBlk] row scales
static_assert(kLds8pScaleFp8 + 2 * kBlk * 4 <= 2 * kTileBytes, "the FP8 row scales stay below the weight area");

// The body of decode_kernel8p for workgroup `block` of its launch, on the LDS
// at `smem` (kLds8pBytes).
template <bool KV_FP8, bool DIRECT, bool PREFETCH>
__device__ __forceinline__ void decode8p_body(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, const DecodeArgs& a, int block, uint8_t* smem) {
  constexpr int kCt = 16;                         // column tiles of 16 owned by a wave
  constexpr int kStagePitch = 512 * 4 + 16;       // LDS pitch of a staged fp32 output row
  static_assert(64 * kStagePitch <= 2 * kTileBytes, "staging must fit in the tile buffers");
  uint8_t* const s_tile = smem;                   // [2 * kTileBytes]
  // Per wave: its block weights (bf16 hi terms at +0, lo terms at +1024, 16
  // bytes a lane in MFMA operand order), read by the partner wave.
  uint8_t (*const s_pex)[2048] = reinterpret_cast<uint8_t (*)[2048]>(smem + 2 * kTileBytes);
  float (*const s_scale)[kBlk] = reinterpret_cast<float (*)[kBlk]>(smem + kLds8pScaleFp8);   // FP8
  constexpr int kQOff = KV_FP8 ? kLds8pQFp8 : kQOffset;     // LDS byte offset of the staged Q rows
  constexpr int kBufBytes = KV_FP8 ? kCodeTileBytes : kTileBytes;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane & 15;               // head within the head tile (MFMA column)
  const int G = lane >> 4;                // k-group of the 16x16x32 operand layout
  const int hq = wave & 3;                // head tile: heads [16 hq, 16 hq + 16)
  const int sg = wave >> 2;               // scores: slots [32 sg, +32); output: columns [256 sg, +256)
  const int head = 16 * hq + hl;
  float* const pex_own = (float*)s_pex[wave];
  const float* const pex_par = (const float*)s_pex[wave ^ 4];

  const Job job = decode_job(block, 0, num_splits, n_blocks, job0, s_q * num_splits);
  if (!job.live) return;                          // padding of the grid (whole workgroup)
  const int t = job.t;
  const int32_t* idx_row = indices + (int64_t)t * topk;

  float M_run = kNoFrame;             // integer frame of this lane's head, shared by the wave pair
  float m_seen = kMaskedScore;        // largest score seen so far over this wave's slots
  float l_run = 0.f;                  // this lane's share of the denominator
  float l_par = 0.f;                  // the partner wave's denominator (after the last pass)
  f32x4 acc[kCt];                     // O^T: column tile ct -> columns 256 sg + 16ct + 4G + i
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (job.b0 < job.b1) {
    const JobIndices ji{idx_row, topk, job.b1, a.n_pool};
    auto load_idx = [&](int b) -> int { return ji.load(b, lane); };
    auto slot_in = [&](int b) -> bool { return ji.slot_in(b, lane); };
    auto valid_of = [&](int idx) -> bool { return ji.valid(idx); };
    const float scale_log2 = a.scale_log2;
    bf16x8 qf[18];                    // Q fragments: head, dims 32ks + 8G .. +8
    const uint32_t tile_lds0 = lds_addr(s_tile);
    bool framed = false;              // workgroup-uniform: the pair frames are set

    // bf16: wave w gathers rows [8w, 8w + 8), lanes 8k..8k+7 one row, chunk
    // (l & 7) ^ (row & 7) of each octet.  FP8: waves 0-3 gather rows
    // [16w, 16w + 16) of the code tile, 4 lanes a row.  A masked row copies the
    // zero row, so a gathering wave always has exactly 9 DMAs in flight (the
    // first pass counts on it).
    const bool gathers = !KV_FP8 || wave < 4;
    auto row_src = [&](int idx_lane) -> const uint8_t* {
      const int row_idx = __shfl(idx_lane, KV_FP8 ? 16 * (wave & 3) + (lane >> 2) : 8 * wave + (lane >> 3));
      return gather_src<KV_FP8>(a, row_idx, valid_of(row_idx), lane);
    };
    auto issue_gather = [&](int idx_lane, int buf) { gather_block8<KV_FP8>(row_src(idx_lane), tile_lds0, buf, wave); };

    // per-lane LDS byte offsets of the operand reads (the tile layout above)
    const int sw_k = rsw(hl);
    const int kb0 = hl * 128 + ((G ^ sw_k) * 16);              // K chunk 4ks + G, ks even
    const int kb1 = hl * 128 + (((4 + G) ^ sw_k) * 16);        // ks odd
    const Fp8Offsets f8 = fp8_offsets(lane);                  // FP8 pool: K and V^T reads of the codes
    const int sw_v = rsw(4 * G + ((lane >> 2) & 3));
    const int vrow = (4 * G + ((lane >> 2) & 3)) * 128 + (lane & 1) * 8;
    int vb[4];                                                  // column tile ct & 3
#pragma unroll
    for (int m = 0; m < 4; ++m) vb[m] = vrow + (((2 * m + ((lane & 3) >> 1)) ^ sw_v) * 16);

    // ---- prologue: Q rows (heads) [8w, 8w + 8) into LDS by wave w, at kQOff
    // (rows of heads >= h_q copy head 0; their results are never stored)
    int idx_cur;
    {
      const int r0 = 8 * wave + (lane >> 3);
      const int chunk = ((lane & 7) ^ rsw(lane >> 3)) * 16;
      const uint8_t* qbase = (const uint8_t*)(q_ptr + (int64_t)t * h_q * 576);
      idx_cur = load_idx_and_q1(idx_row + min(job.b0 * kBlk + lane, topk - 1),
                                qbase + (int64_t)(r0 < h_q ? r0 : 0) * 1152 + chunk,
                                __builtin_amdgcn_readfirstlane(tile_lds0 + kQOff + wave * 1024));
    }

    auto run_pass = [&](const bool first) __attribute__((always_inline)) -> bool {
    bool overflow = false;
    if (!first) idx_cur = load_idx(job.b0);
    idx_cur = slot_in(job.b0) ? idx_cur : -1;
    issue_gather(idx_cur, 0);
    int idx_nxt = load_idx(job.b0 + 1);
    bool valid_cur = valid_of(idx_cur);
    if (first) {
      // Q rows landed (issued first; block b0's 9 DMAs of a gathering wave
      // and, with the look-ahead, the next index load stay in flight).
      if (gathers)
        wait_q_rows<PREFETCH, 9>();
      else
        wait_q_rows<PREFETCH, 0>();
      lds_barrier();
      load_q_frags(qf, lds_addr(s_tile) + kQOff + hq * 2048, kb0, kb1);
    }
    // FP8: block b0's row scales (stored by wave 0 at the top of the block loop).
    float sc_cur = (KV_FP8 && wave == 0 && valid_cur) ? a.kv_scale[idx_cur] : 0.f;

    for (int b = job.b0; b < job.b1; ++b) {
      const int cur = (b - job.b0) & 1;
      wait_vmem_all();          // this wave's share of block b has landed
      if (KV_FP8 && wave == 0) s_scale[cur][lane] = sc_cur;
      lds_barrier();            // ... and every wave's; block b-1 and its weights fully consumed
      // slot s of the block is valid iff bit s is set (the same in every wave)
      const uint32_t vhalf = (uint32_t)(__ballot(valid_cur) >> (32 * sg));
      const bool blk_any = __ballot(valid_cur) != 0ull;

      // Block b+1: one DMA per QK^T k-step pair (masked rows and rows past the
      // job's last block copy the zero row).
      bool valid_nxt = false;
      float sc_nxt = 0.f;
      const uint8_t* gsrc = g_zero_row;
      uint32_t gbase = 0u;
      if (PREFETCH) {
        idx_nxt = slot_in(b + 1) ? idx_nxt : -1;
        valid_nxt = valid_of(idx_nxt);
        if (KV_FP8 && wave == 0 && valid_nxt) sc_nxt = a.kv_scale[idx_nxt];
        gsrc = row_src(idx_nxt);
        gbase = __builtin_amdgcn_readfirstlane(tile_lds0 + (cur ^ 1) * kBufBytes + (KV_FP8 ? (wave & 3) : wave) * 1024);
      }
      auto gather_dma = [&](const int d) __attribute__((always_inline)) {
        if (!PREFETCH || !gathers) return;
        constexpr int L = KV_FP8 ? 4096 : 8192, Gs = KV_FP8 ? 64 : 128;
        switch (d) {
          case 0: dma_one<L, Gs, 0>(gsrc, gbase); break;
          case 1: dma_one<L, Gs, 1>(gsrc, gbase); break;
          case 2: dma_one<L, Gs, 2>(gsrc, gbase); break;
          case 3: dma_one<L, Gs, 3>(gsrc, gbase); break;
          case 4: dma_one<L, Gs, 4>(gsrc, gbase); break;
          case 5: dma_one<L, Gs, 5>(gsrc, gbase); break;
          case 6: dma_one<L, Gs, 6>(gsrc, gbase); break;
          case 7: dma_one<L, Gs, 7>(gsrc, gbase); break;
          default: dma_one<L, Gs, 8>(gsrc, gbase); break;
        }
      };
      const int idx_after = load_idx(b + 2);

      // Block b's operands: bf16 rows, or the e4m3 codes converted in registers.
      const uint32_t tl = lds_addr(s_tile + cur * kBufBytes);
      uint32_t kbase[4], vbase[4];
      if constexpr (KV_FP8) {
        kbase[0] = opaque(tl + f8.k[0]);
        kbase[1] = opaque(tl + f8.k[1]);
        kbase[2] = kbase[3] = 0u;
        const uint32_t tlv = tl + sg * 4 * 4096;     // this wave's 256 columns
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + f8.v[m]);
      } else {
        kbase[0] = opaque(tl + kb0);
        kbase[1] = opaque(tl + kb1);
        kbase[2] = opaque(tl + kb0 + 65536);
        kbase[3] = opaque(tl + kb1 + 65536);
        const uint32_t tlv = tl + sg * 4 * 8192;     // this wave's 256 columns
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + vb[m]);
      }
      auto kfrag = [&](int ks, int st) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_kfrag(kbase[ks & 1] + (ks >> 1) * 4096 + st * 1024);
        const uint32_t kp = kbase[(ks & 1) + (ks >= 16 ? 2 : 0)] + ((ks >> 1) & 7) * 8192 + st * 2048;
        return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)kp;
      };
      auto vfrag = [&](int ct, int kk) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_vfrag(vbase[ct & 3] + (ct >> 2) * 4096 + kk * 2048);
        const uint32_t vp = vbase[ct & 3] + (ct >> 2) * 8192 + kk * 4096;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)vp);
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)(vp + 2048));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
        return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
      };

      // ---- S^T = K . Q^T over this wave's 2 slot tiles (2 sg, 2 sg + 1)
      constexpr int kAheadK = 2, kRing = kAheadK + 2, kAheadV = 4;
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      {
        bf16x8 kf[kRing][2];
#pragma unroll
        for (int a0 = 0; a0 < kAheadK; ++a0)
#pragma unroll
          for (int u = 0; u < 2; ++u) kf[a0][u] = kfrag(a0, 2 * sg + u);
#pragma unroll
        for (int j = 0; j < 9; ++j) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int ka = 2 * j + e + kAheadK;
            if (ka < 18) {
#pragma unroll
              for (int u = 0; u < 2; ++u) kf[ka % kRing][u] = kfrag(ka, 2 * sg + u);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int ks = 2 * j + e;
              sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % kRing][u], qf[ks], sacc[u], 0, 0, 0);
            }
          gather_dma(j);                // the next block's DMAs 0..8, one per k-step pair
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax of this wave's 32 slots (lane: slots 32 sg + 16u + 4G + i).
      // The first V^T fragments of the PV over these slots are requested first.
      bf16x8 vf[kAheadV + 1];
#pragma unroll
      for (int a0 = 0; a0 < kAheadV; ++a0) vf[a0] = vfrag(a0, sg);
      const uint32_t vbits = vhalf >> (4 * G);
      f32x4 rsc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (KV_FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) rsc[u] = *(const f32x4*)&s_scale[cur][32 * sg + 16 * u + 4 * G];
      }
      float tv[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bias = ((vbits >> (16 * u + i)) & 1u) ? 0.f : kMaskedScore;
          tv[4 * u + i] = KV_FP8 ? fmaf(sacc[u][i] * scale_log2, rsc[u][i], bias) : fmaf(sacc[u][i], scale_log2, bias);
        }
      float m = fmaxf(fmaxf(fmaxf(tv[0], tv[1]), fmaxf(tv[2], tv[3])), fmaxf(fmaxf(tv[4], tv[5]), fmaxf(tv[6], tv[7])));
      m = rows_max(m);
      m_seen = fmaxf(m_seen, m);
      if (!framed && blk_any) {
        // first block with a valid slot: the pair's frame is the floor of the
        // larger of the two halves' maxima
        if (G == 0) pex_own[hl] = m;
        lds_barrier();
        M_run = floorf(fmaxf(m, pex_par[hl]));
        framed = true;
        lds_barrier();          // the partner has read m before the weights overwrite it
      }
      overflow |= m > M_run + kFrameSlack;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float tt = tv[e];
        float p = __builtin_amdgcn_exp2f(tt - M_run);
        l_run += p;
        if (KV_FP8) p *= rsc[e >> 2][e & 3];
        pv[e] = p;
      }
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t h2 = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
        ph[j] = h2;
        pl[j] = pack_bf16x2(pv[2 * j] - __uint_as_float(h2 << 16), pv[2 * j + 1] - __uint_as_float(h2 & 0xFFFF0000u));
      }
      const bf16x8 pfh = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
      *(bf16x8*)(s_pex[wave] + 16 * lane) = pfh;
      *(bf16x8*)(s_pex[wave] + 1024 + 16 * lane) = pfl;

      // ---- O^T += V^T . P^T: this wave's slots (k-step sg), then the partner's
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        if (ct + kAheadV < kCt) vf[(ct + kAheadV) % (kAheadV + 1)] = vfrag(ct + kAheadV, sg);
        __builtin_amdgcn_sched_barrier(0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct % (kAheadV + 1)], pfh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct % (kAheadV + 1)], pfl, acc[ct], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 vg[kAheadV + 1];
#pragma unroll
      for (int a0 = 0; a0 < kAheadV; ++a0) vg[a0] = vfrag(a0, sg ^ 1);
      lds_barrier();            // every wave's weights are in LDS
      const bf16x8 qfh = *(const bf16x8*)(s_pex[wave ^ 4] + 16 * lane);
      const bf16x8 qfl = *(const bf16x8*)(s_pex[wave ^ 4] + 1024 + 16 * lane);
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        if (ct + kAheadV < kCt) vg[(ct + kAheadV) % (kAheadV + 1)] = vfrag(ct + kAheadV, sg ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vg[ct % (kAheadV + 1)], qfh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vg[ct % (kAheadV + 1)], qfl, acc[ct], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      valid_cur = valid_nxt;
      sc_cur = sc_nxt;
      idx_nxt = idx_after;
    }
    wait_vmem_all();            // the last block's look-ahead gather lands before LDS is reused
    return overflow;
    };

    // End of a pass: every wave posts its largest score, its denominator and
    // its overflow flag; returns whether any wave of the workgroup overflowed.
    auto end_exchange = [&](const bool overflow) __attribute__((always_inline)) -> bool {
      const bool any_ov = post_pass<kWaves8>(overflow, m_seen, l_run, pex_own, s_pex[0], 2048, hl, G, lane);
      l_par = pex_par[16 + hl];
      return any_ov;
    };

    if (end_exchange(run_pass(true))) {
      // the frame of the pair's largest score bounds every weight by 2
      const float ms = fmaxf(m_seen, pex_par[hl]);
      M_run = ms > kMaskedScore ? floorf(ms) : kNoFrame;
      framed = true;
      l_run = 0.f;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      end_exchange(run_pass(false));
    }
  }

  // ---- epilogue: l = both halves' denominators (one frame), O = acc / l ----
  const bool head_ok = head < h_q;                // fewer heads (a direct FP8 output): rows past h_q are padding
  const float l = l_run + l_par;
  const bool any = l > 0.f;
  const float lse = any ? M_run + __builtin_amdgcn_logf(l) : kNegInf;
  float oscale = any ? 1.0f / l : 0.f;
  if (DIRECT && a.sink != nullptr && any && head_ok) {
    const float z = a.sink[head] * kLog2e - lse;
    oscale = oscale / (1.0f + __builtin_amdgcn_exp2f(z));
  }
  const int64_t rowt = DIRECT ? (int64_t)t * h_q : ((int64_t)job.s * s_q + t) * h_q;
  if (sg == 0 && G == 0 && head_ok) {
    if (!DIRECT)
      a.lse_accum[rowt + head] = lse;
    else if (a.lse_out != nullptr)
      a.lse_out[rowt + head] = lse;
  }

  // Staging (row = head, the tiles are free): wave (hq, sg) writes its 16
  // heads x 256 columns; after the barrier wave w stores heads [8w, 8w + 8)
  // in whole rows.  A direct FP8 output takes the token's amax over every
  // head and column on the way (through a word of the weight area that the
  // end-of-pass exchange does not read).
  const bool fp8_out = DIRECT && a.out_dtype == kOutFp8;
  float* const s_red = (float*)(s_pex[0] + 1024);  // [kWaves8]
  float amax = 0.f;
  {
    uint8_t* stg = s_tile + head * kStagePitch + (256 * sg + 4 * G) * 4;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      const f32x4 v = acc[ct] * oscale;
      if (fp8_out && head_ok)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      *(f32x4*)(stg + 64 * ct) = v;
    }
  }
  if (fp8_out) {
    amax = wave_max(amax);
    if (lane == 0) s_red[wave] = amax;
  }
  lds_barrier();
  float qscale = 1.0f;
  if (fp8_out) {
    amax = fmaxf(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])),
                 fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7])));
    qscale = amax > 0.f ? amax / 448.0f : 1.0f;
    if (tid == 0) a.out_scale[t] = qscale;
  }
  const uint8_t* st = s_tile + 8 * wave * kStagePitch;
  const int64_t row0 = rowt + 8 * wave;
  if (8 * wave < h_q) {                          // (h_q is a multiple of 16)
    if (!DIRECT || a.out_dtype == kOutF32) {     // 1 KB of one row per instruction
      float* dst = (DIRECT ? (float*)a.out : a.o_accum) + row0 * 512;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = j >> 1, c = 256 * (j & 1) + 4 * lane;
        *(f32x4*)(dst + r * 512 + c) = *(const f32x4*)(st + r * kStagePitch + 4 * c);
      }
    } else if (a.out_dtype == kOutBf16) {        // 1 KB of one row per instruction
      uint16_t* dst = (uint16_t*)a.out + row0 * 512 + 8 * lane;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const f32x4 v0 = *(const f32x4*)(st + r * kStagePitch + 32 * lane);
        const f32x4 v1 = *(const f32x4*)(st + r * kStagePitch + 32 * lane + 16);
        *(u32x4*)(dst + r * 512) = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                         pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
      }
    } else {                                     // e4m3: two 512 B rows per instruction
      uint8_t* dst = (uint8_t*)a.out + row0 * 512;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 2 * j + (lane >> 5);
        const uint8_t* src = st + r * kStagePitch + 64 * (lane & 31);
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 v = *(const f32x4*)(src + 16 * k);
          w[k] = e4m3_encode(v[0] / qscale) | (e4m3_encode(v[1] / qscale) << 8) |
                 (e4m3_encode(v[2] / qscale) << 16) | (e4m3_encode(v[3] / qscale) << 24);
        }
        *(u32x4*)(dst + r * 512 + 16 * (lane & 31)) = w;
      }
    }
  }
  // Split jobs of a decode with an FP8 output: seed the combine's amax and counters.
  if (!DIRECT && a.out_scale != nullptr && job.s == 0 && tid == 0) seed_fp8_combine(a.out_scale, a.out, t, h_q);
}

template <bool KV_FP8, bool DIRECT, bool PREFETCH>
__global__ __launch_bounds__(kThreads8) void decode_kernel8p(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds8pBytes];
  decode8p_body<KV_FP8, DIRECT, PREFETCH>(indices, q_ptr, num_splits, n_blocks, s_q, topk, h_q, job0, a,
                                          (int)blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// decode8h_body: a job in two workgroups that each own 32 of its 64 heads and
// all 512 output columns.  Unlike two column parts would, the two head
// parts do not repeat each other's QK^T.  Wave w owns
// head tile w & 1 (heads 32 part + 16 (w & 1) .. +15) and scores slot quarter
// w >> 1 (16 slots) of every block; the four waves of a head tile trade their
// bf16 weights through LDS, and each accumulates every slot of the block into
// its own quarter of the columns (128).  The four share one integer frame per
// head, agreed on as in decode_kernel8p.  The job's two workgroups are 8 block
// ids apart (one XCD, one L2 for the gathered rows).  KV_FP8: waves 0-3
// gather the e4m3 code tile (wave w: rows [16w, +16)), every wave reads its
// operands from the codes, and the row scale multiplies the score after QK^T
// and the weight before PV.
// ---------------------------------------------------------------------------
// LDS of decode8h_body: the two tiles (FP8: two code tiles), the weight
// exchange (1 KB a wave), then the per-block row scales.
constexpr int kLds8hScale = 2 * kTileBytes + kWaves8 * 1024;
constexpr int kLds8hBytes = kLds8hScale + 2 * kBlk * 4;

template <bool KV_FP8, bool DIRECT, bool PREFETCH>
__device__ __forceinline__ void decode8h_body(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, const DecodeArgs& a, int block, uint8_t* smem) {
  constexpr int kCt = 8;                          // column tiles of 16 owned by a wave
  constexpr int kStagePitch = 512 * 4 + 16;       // LDS pitch of a staged fp32 output row
  static_assert(32 * kStagePitch <= 2 * kTileBytes, "staging must fit in the tile buffers");
  uint8_t* const s_tile = smem;                   // [2 * kTileBytes]
  // Per wave: its block weights (4 a lane, MFMA output order): bf16 hi terms
  // at +0, lo terms at +512, 8 bytes a lane.
  uint8_t (*const s_pex)[1024] = reinterpret_cast<uint8_t (*)[1024]>(smem + 2 * kTileBytes);
  float (*const s_scale)[kBlk] = reinterpret_cast<float (*)[kBlk]>(smem + kLds8hScale);   // [2][kBlk] (FP8)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane & 15;               // head within the head tile (MFMA column)
  const int G = lane >> 4;                // k-group of the 16x16x32 operand layout
  const int hq = wave & 1;                // head tile within the part
  const int sq = wave >> 1;               // scores: slots [16 sq, +16); output: columns [128 sq, +128)
  float* const pex_own = (float*)s_pex[wave];
  auto pex_of = [&](int q) -> const float* { return (const float*)s_pex[hq + 2 * q]; };   // quarter q's wave

  const Job job = decode_job(block, 1, num_splits, n_blocks, job0, s_q * num_splits);
  if (!job.live) return;                          // padding of the grid (whole workgroup)
  const int t = job.t;
  const int hbase = 32 * job.part;                // first head of this part
  const int hloc = 16 * hq + hl;                  // head within the part
  const int head = hbase + hloc;
  const int32_t* idx_row = indices + (int64_t)t * topk;

  float M_run = kNoFrame;             // integer frame of this lane's head, shared by the four waves
  float m_seen = kMaskedScore;        // largest score seen so far over this wave's slots
  float l_run = 0.f;                  // this lane's share of the denominator
  float l_tot = 0.f;                  // the head's denominator over all four quarters (after the last pass)
  f32x4 acc[kCt];                     // O^T: column tile ct -> columns 128 sq + 16ct + 4G + i
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (job.b0 < job.b1) {
    const JobIndices ji{idx_row, topk, job.b1, a.n_pool};
    auto load_idx = [&](int b) -> int { return ji.load(b, lane); };
    auto slot_in = [&](int b) -> bool { return ji.slot_in(b, lane); };
    auto valid_of = [&](int idx) -> bool { return ji.valid(idx); };
    const float scale_log2 = a.scale_log2;
    bf16x8 qf[18];                    // Q fragments: head, dims 32ks + 8G .. +8
    const uint32_t tile_lds0 = lds_addr(s_tile);
    bool framed = false;              // workgroup-uniform: the frames are set

    // bf16: wave w gathers rows [8w, 8w + 8) (as decode_kernel8p); FP8: waves
    // 0-3 gather rows [16w, 16w + 16) of the code tile, 4 lanes a row.  9 DMAs
    // a gathering wave, a masked row copying the zero row.
    const bool gathers = !KV_FP8 || wave < 4;
    auto row_src = [&](int idx_lane) -> const uint8_t* {
      const int row_idx = __shfl(idx_lane, KV_FP8 ? 16 * (wave & 3) + (lane >> 2) : 8 * wave + (lane >> 3));
      return gather_src<KV_FP8>(a, row_idx, valid_of(row_idx), lane);
    };
    auto issue_gather = [&](int idx_lane, int buf) { gather_block8<KV_FP8>(row_src(idx_lane), tile_lds0, buf, wave); };

    // per-lane LDS byte offsets of the operand reads (the tile layout above)
    const int sw_k = rsw(hl);
    const int kb0 = hl * 128 + ((G ^ sw_k) * 16);              // K chunk 4ks + G, ks even
    const int kb1 = hl * 128 + (((4 + G) ^ sw_k) * 16);        // ks odd
    const Fp8Offsets f8 = fp8_offsets(lane);                  // FP8 pool: K and V^T reads of the codes
    const int sw_v = rsw(4 * G + ((lane >> 2) & 3));
    const int vrow = (4 * G + ((lane >> 2) & 3)) * 128 + (lane & 1) * 8;
    int vb[4];                                                  // column tile ct & 3
#pragma unroll
    for (int m = 0; m < 4; ++m) vb[m] = vrow + (((2 * m + ((lane & 3) >> 1)) ^ sw_v) * 16);

    // ---- prologue: the part's 32 Q rows into LDS at kQOffset; wave w stages
    // rows [8 (w & 3), +8) (waves 4-7 repeat waves 0-3's rows, same bytes, so
    // every wave has the same loads in flight).
    int idx_cur;
    {
      const int r0 = 8 * (wave & 3) + (lane >> 3);
      const int chunk = ((lane & 7) ^ rsw(lane >> 3)) * 16;
      const uint8_t* qbase = (const uint8_t*)(q_ptr + ((int64_t)t * h_q + hbase) * 576);
      idx_cur = load_idx_and_q1(idx_row + min(job.b0 * kBlk + lane, topk - 1), qbase + (int64_t)r0 * 1152 + chunk,
                                __builtin_amdgcn_readfirstlane(tile_lds0 + kQOffset + (wave & 3) * 1024));
    }

    auto run_pass = [&](const bool first) __attribute__((always_inline)) -> bool {
    bool overflow = false;
    if (!first) idx_cur = load_idx(job.b0);
    idx_cur = slot_in(job.b0) ? idx_cur : -1;
    issue_gather(idx_cur, 0);
    int idx_nxt = load_idx(job.b0 + 1);
    bool valid_cur = valid_of(idx_cur);
    if (first) {
      // Q rows landed (issued first; block b0's 9 DMAs of a gathering wave
      // and, with the look-ahead, the next index load stay in flight).
      if (gathers)
        wait_q_rows<PREFETCH, 9>();
      else
        wait_q_rows<PREFETCH, 0>();
      lds_barrier();
      load_q_frags(qf, lds_addr(s_tile) + kQOffset + hq * 2048, kb0, kb1);
    }
    // FP8: block b0's row scales (stored at the top of the block loop).
    float sc_cur = (KV_FP8 && valid_cur) ? a.kv_scale[idx_cur] : 0.f;

    for (int b = job.b0; b < job.b1; ++b) {
      const int cur = (b - job.b0) & 1;
      wait_vmem_all();          // this wave's share of block b has landed
      if (KV_FP8 && wave == 0) s_scale[cur][lane] = sc_cur;
      lds_barrier();            // ... and every wave's; block b-1 and its weights fully consumed
      // slot s of the block is valid iff bit s is set (the same in every wave)
      const uint64_t vmask = __ballot(valid_cur);
      const uint32_t vquart = (uint32_t)(vmask >> (16 * sq));
      const bool blk_any = vmask != 0ull;

      // Block b+1: one DMA per QK^T k-step pair (masked rows and rows past the
      // job's last block copy the zero row).
      bool valid_nxt = false;
      float sc_nxt = 0.f;
      const uint8_t* gsrc = g_zero_row;
      uint32_t gbase = 0u;
      if (PREFETCH) {
        idx_nxt = slot_in(b + 1) ? idx_nxt : -1;
        valid_nxt = valid_of(idx_nxt);
        if (KV_FP8 && wave == 0 && valid_nxt) sc_nxt = a.kv_scale[idx_nxt];
        gsrc = row_src(idx_nxt);
        gbase = __builtin_amdgcn_readfirstlane(tile_lds0 + (cur ^ 1) * (KV_FP8 ? kCodeTileBytes : kTileBytes) +
                                               (KV_FP8 ? (wave & 3) : wave) * 1024);
      }
      auto gather_dma = [&](const int d) __attribute__((always_inline)) {
        if (!PREFETCH || !gathers) return;
        constexpr int L = KV_FP8 ? 4096 : 8192, Gs = KV_FP8 ? 64 : 128;
        switch (d) {
          case 0: dma_one<L, Gs, 0>(gsrc, gbase); break;
          case 1: dma_one<L, Gs, 1>(gsrc, gbase); break;
          case 2: dma_one<L, Gs, 2>(gsrc, gbase); break;
          case 3: dma_one<L, Gs, 3>(gsrc, gbase); break;
          case 4: dma_one<L, Gs, 4>(gsrc, gbase); break;
          case 5: dma_one<L, Gs, 5>(gsrc, gbase); break;
          case 6: dma_one<L, Gs, 6>(gsrc, gbase); break;
          case 7: dma_one<L, Gs, 7>(gsrc, gbase); break;
          default: dma_one<L, Gs, 8>(gsrc, gbase); break;
        }
      };
      const int idx_after = load_idx(b + 2);

      // Block b's operands: bf16 rows, or the e4m3 codes converted in registers.
      const uint32_t tl = lds_addr(s_tile + cur * (KV_FP8 ? kCodeTileBytes : kTileBytes));
      uint32_t kbase[4], vbase[4];
      if constexpr (KV_FP8) {
        kbase[0] = opaque(tl + f8.k[0]);
        kbase[1] = opaque(tl + f8.k[1]);
        kbase[2] = kbase[3] = 0u;
        const uint32_t tlv = tl + sq * 2 * 4096;     // this wave's 128 columns
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + f8.v[m]);
      } else {
        kbase[0] = opaque(tl + kb0);
        kbase[1] = opaque(tl + kb1);
        kbase[2] = opaque(tl + kb0 + 65536);
        kbase[3] = opaque(tl + kb1 + 65536);
        const uint32_t tlv = tl + sq * 2 * 8192;
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + vb[m]);
      }
      auto kfrag = [&](int ks, int st) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_kfrag(kbase[ks & 1] + (ks >> 1) * 4096 + st * 1024);
        const uint32_t kp = kbase[(ks & 1) + (ks >= 16 ? 2 : 0)] + ((ks >> 1) & 7) * 8192 + st * 2048;
        return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)kp;
      };
      auto vfrag = [&](int ct, int kk) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_vfrag(vbase[ct & 3] + (ct >> 2) * 4096 + kk * 2048);
        const uint32_t vp = vbase[ct & 3] + (ct >> 2) * 8192 + kk * 4096;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)vp);
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)(vp + 2048));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
        return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
      };

      // ---- S^T = K . Q^T over this wave's slot tile (sq): one accumulator
      constexpr int kAheadK = 3, kRing = kAheadK + 1, kAheadV = 4;
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        bf16x8 kf[kRing];
#pragma unroll
        for (int a0 = 0; a0 < kAheadK; ++a0) kf[a0] = kfrag(a0, sq);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if (ks + kAheadK < 18) kf[(ks + kAheadK) % kRing] = kfrag(ks + kAheadK, sq);
          __builtin_amdgcn_sched_barrier(0);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % kRing], qf[ks], sacc, 0, 0, 0);
          if (ks & 1) gather_dma(ks >> 1);   // the next block's DMAs 0..8, one per k-step pair
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax of this wave's 16 slots (lane: slots 16 sq + 4G + i)
      bf16x8 vf[kAheadV + 1];
#pragma unroll
      for (int a0 = 0; a0 < kAheadV; ++a0) vf[a0] = vfrag(a0, 0);
      const uint32_t vbits = vquart >> (4 * G);
      f32x4 rsc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (KV_FP8) rsc = *(const f32x4*)&s_scale[cur][16 * sq + 4 * G];
      float tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bias = ((vbits >> i) & 1u) ? 0.f : kMaskedScore;
        tv[i] = KV_FP8 ? fmaf(sacc[i] * scale_log2, rsc[i], bias) : fmaf(sacc[i], scale_log2, bias);
      }
      float m = fmaxf(fmaxf(tv[0], tv[1]), fmaxf(tv[2], tv[3]));
      m = rows_max(m);
      m_seen = fmaxf(m_seen, m);
      if (!framed && blk_any) {
        // first block with a valid slot: the frame is the floor of the largest
        // of the four quarters' maxima
        if (G == 0) pex_own[hl] = m;
        lds_barrier();
        M_run = floorf(fmaxf(fmaxf(pex_of(0)[hl], pex_of(1)[hl]), fmaxf(pex_of(2)[hl], pex_of(3)[hl])));
        framed = true;
        lds_barrier();          // every wave has read the maxima before the weights overwrite them
      }
      overflow |= m > M_run + kFrameSlack;
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float tt = tv[e];
        float p = __builtin_amdgcn_exp2f(tt - M_run);
        l_run += p;
        if (KV_FP8) p *= rsc[e];
        pv[e] = p;
      }
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t h2 = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
        ph[j] = h2;
        pl[j] = pack_bf16x2(pv[2 * j] - __uint_as_float(h2 << 16), pv[2 * j + 1] - __uint_as_float(h2 & 0xFFFF0000u));
      }
      *(u32x2*)(s_pex[wave] + 8 * lane) = u32x2{ph[0], ph[1]};
      *(u32x2*)(s_pex[wave] + 512 + 8 * lane) = u32x2{pl[0], pl[1]};
      lds_barrier();            // every wave's weights are in LDS

      // ---- O^T += V^T . P^T over the block: k-step kk takes the weights of
      // quarters 2kk (its first 4 k-indices of each group) and 2kk + 1.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2 h0 = *(const u32x2*)(s_pex[hq + 4 * kk] + 8 * lane);
        const u32x2 h1 = *(const u32x2*)(s_pex[hq + 4 * kk + 2] + 8 * lane);
        const u32x2 l0 = *(const u32x2*)(s_pex[hq + 4 * kk] + 512 + 8 * lane);
        const u32x2 l1 = *(const u32x2*)(s_pex[hq + 4 * kk + 2] + 512 + 8 * lane);
        const bf16x8 pfh = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
        const bf16x8 pfl = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          const int n = kCt * kk + ct;            // position in the fragment stream
          if (n + kAheadV < 2 * kCt)
            vf[(n + kAheadV) % (kAheadV + 1)] = vfrag((n + kAheadV) % kCt, (n + kAheadV) / kCt);
          __builtin_amdgcn_sched_barrier(0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n % (kAheadV + 1)], pfh, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n % (kAheadV + 1)], pfl, acc[ct], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      valid_cur = valid_nxt;
      sc_cur = sc_nxt;
      idx_nxt = idx_after;
    }
    wait_vmem_all();            // the last block's look-ahead gather lands before LDS is reused
    return overflow;
    };

    // End of a pass: every wave posts its largest score, its denominator and
    // its overflow flag; returns whether any wave of the workgroup overflowed.
    auto end_exchange = [&](const bool overflow) __attribute__((always_inline)) -> bool {
      const bool any_ov = post_pass<kWaves8>(overflow, m_seen, l_run, pex_own, s_pex[0], 1024, hl, G, lane);
      // the same sum, in the same order, in each of the head tile's four waves
      l_tot = ((pex_of(0)[16 + hl] + pex_of(1)[16 + hl]) + pex_of(2)[16 + hl]) + pex_of(3)[16 + hl];
      return any_ov;
    };

    if (end_exchange(run_pass(true))) {
      // the frame of the largest score of the four quarters bounds every weight by 2
      const float ms = fmaxf(fmaxf(pex_of(0)[hl], pex_of(1)[hl]), fmaxf(pex_of(2)[hl], pex_of(3)[hl]));
      M_run = ms > kMaskedScore ? floorf(ms) : kNoFrame;
      framed = true;
      l_run = 0.f;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      end_exchange(run_pass(false));
    }
  }

  // ---- epilogue: l = the four quarters' denominators (one frame), O = acc / l
  const float l = l_tot;
  const bool any = l > 0.f;
  const float lse = any ? M_run + __builtin_amdgcn_logf(l) : kNegInf;
  float oscale = any ? 1.0f / l : 0.f;
  if (DIRECT && a.sink != nullptr && any) {
    const float z = a.sink[head] * kLog2e - lse;
    oscale = oscale / (1.0f + __builtin_amdgcn_exp2f(z));
  }
  const int64_t rowt = (DIRECT ? (int64_t)t * h_q : ((int64_t)job.s * s_q + t) * h_q) + hbase;
  if (sq == 0 && G == 0) {
    if (!DIRECT)
      a.lse_accum[rowt + hloc] = lse;
    else if (a.lse_out != nullptr)
      a.lse_out[rowt + hloc] = lse;
  }

  // Staging (row = head of the part, the tiles are free): wave (hq, sq) writes
  // its 16 heads x 128 columns; after the barrier wave w stores heads
  // [4w, 4w + 4) of the part in whole rows.
  {
    uint8_t* stg = s_tile + hloc * kStagePitch + (128 * sq + 4 * G) * 4;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) *(f32x4*)(stg + 64 * ct) = acc[ct] * oscale;
  }
  lds_barrier();
  const uint8_t* st = s_tile + 4 * wave * kStagePitch;
  const int64_t row0 = rowt + 4 * wave;
  if (!DIRECT || a.out_dtype == kOutF32) {       // 1 KB of one row per instruction
    float* dst = (DIRECT ? (float*)a.out : a.o_accum) + row0 * 512;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j >> 1, c = 256 * (j & 1) + 4 * lane;
      *(f32x4*)(dst + r * 512 + c) = *(const f32x4*)(st + r * kStagePitch + 4 * c);
    }
  } else {                                       // bf16 (a direct FP8 output never takes this kernel)
    uint16_t* dst = (uint16_t*)a.out + row0 * 512 + 8 * lane;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 v0 = *(const f32x4*)(st + r * kStagePitch + 32 * lane);
      const f32x4 v1 = *(const f32x4*)(st + r * kStagePitch + 32 * lane + 16);
      *(u32x4*)(dst + r * 512) = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                       pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
    }
  }
  // Split jobs of a decode with an FP8 output: seed the combine's amax and counters.
  if (!DIRECT && a.out_scale != nullptr && job.s == 0 && job.part == 0 && tid == 0)
    seed_fp8_combine(a.out_scale, a.out, t, h_q);
}

template <bool KV_FP8, bool DIRECT, bool PREFETCH>
__global__ __launch_bounds__(kThreads8) void decode_kernel8h(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds8hBytes];
  decode8h_body<KV_FP8, DIRECT, PREFETCH>(indices, q_ptr, num_splits, n_blocks, s_q, topk, h_q, job0, a,
                                          (int)blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// decode4t_body: a job in (h_q / 16) * CP workgroups of 4 waves, each owning
// one head tile (16 heads) and 512 / CP of the output columns (CP = 1, 2 or
// 4).  None of them repeats another head tile's QK^T, where column parts of
// every head would each compute all of the heads' scores.  Wave w scores slot quarter
// w (16 slots) of every block; the four waves trade their bf16 weights through
// LDS (as decode8h_body's head tile) and each accumulates every slot into its
// quarter of the workgroup's columns.  One frame per head for the four.  The
// workgroups of a job are 8 block ids apart (one XCD, one L2 for the rows).
// KV_FP8: the e4m3 code tile is gathered (wave w: rows [16w, +16)), the
// operands are read from the codes, and the row scale multiplies the score
// after QK^T and the weight before PV.
// ---------------------------------------------------------------------------
// LDS of decode4t_body: the two tiles (FP8: two code tiles), the weight
// exchange (1 KB a wave), then the per-block row scales (FP8).
constexpr int kLds4tScale = 2 * kTileBytes + kWaves * 1024;
constexpr int kLds4tBytes = kLds4tScale + 2 * kBlk * 4;

template <bool KV_FP8, bool DIRECT, bool PREFETCH, int CP>
__device__ __forceinline__ void decode4t_body(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, const DecodeArgs& a, int block, uint8_t* smem) {
  static_assert(CP == 1 || CP == 2 || CP == 4, "one head tile takes 1, 2 or 4 column parts");
  constexpr int kCols = 512 / CP;                 // columns of the workgroup
  constexpr int kWCols = kCols / 4;               // columns of a wave
  constexpr int kCt = kWCols / 16;                // column tiles of 16 owned by a wave
  constexpr int kStagePitch = kCols * 4 + 16;     // LDS pitch of a staged fp32 output row
  uint8_t* const s_tile = smem;                   // [2 * kTileBytes]
  // Per wave: its block weights (4 a lane, MFMA output order): bf16 hi terms
  // at +0, lo terms at +512, 8 bytes a lane.
  uint8_t (*const s_pex)[1024] = reinterpret_cast<uint8_t (*)[1024]>(smem + 2 * kTileBytes);
  float (*const s_scale)[kBlk] = reinterpret_cast<float (*)[kBlk]>(smem + kLds4tScale);   // [2][kBlk] (FP8)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;              // slot quarter of the scores; column quarter of the output
  const int lane = tid & 63;
  const int hl = lane & 15;               // head within the head tile (MFMA column)
  const int G = lane >> 4;                // k-group of the 16x16x32 operand layout
  float* const pex_own = (float*)s_pex[wave];
  auto pex_of = [&](int q) -> const float* { return (const float*)s_pex[q]; };

  constexpr int kLgCP = CP == 4 ? 2 : CP == 2 ? 1 : 0;
  const int lg_tiles = h_q == 64 ? 2 : h_q == 32 ? 1 : 0;     // h_q / 16 head tiles
  const Job job = decode_job(block, lg_tiles + kLgCP, num_splits, n_blocks, job0, s_q * num_splits);
  if (!job.live) return;                          // padding of the grid (whole workgroup)
  const int t = job.t;
  const int htile = job.part >> kLgCP;            // head tile: heads [16 htile, +16)
  const int cpart = job.part & (CP - 1);          // columns [kCols cpart, +kCols)
  const int head = 16 * htile + hl;
  const int32_t* idx_row = indices + (int64_t)t * topk;

  float M_run = kNoFrame;             // integer frame of this lane's head, shared by the four waves
  float m_seen = kMaskedScore;        // largest score seen so far over this wave's slots
  float l_run = 0.f;                  // this lane's share of the denominator
  float l_tot = 0.f;                  // the head's denominator over all four quarters (after the last pass)
  f32x4 acc[kCt];                     // O^T: column tile ct -> columns kCols cpart + kWCols wave + 16ct + 4G + i
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (job.b0 < job.b1) {
    const JobIndices ji{idx_row, topk, job.b1, a.n_pool};
    auto load_idx = [&](int b) -> int { return ji.load(b, lane); };
    auto slot_in = [&](int b) -> bool { return ji.slot_in(b, lane); };
    auto valid_of = [&](int idx) -> bool { return ji.valid(idx); };
    const float scale_log2 = a.scale_log2;
    bf16x8 qf[18];                    // Q fragments: head, dims 32ks + 8G .. +8
    const uint32_t tile_lds0 = lds_addr(s_tile);
    bool framed = false;              // workgroup-uniform: the frames are set

    // Wave w gathers rows [16w, 16w + 16), a masked row copying the zero row.
    // bf16: two groups of 8 (lanes 8k..8k+7 one row, chunk (l & 7) ^ (row & 7)
    // of each octet), 18 DMAs a wave.  FP8: 4 lanes a row (chunk l & 3 of each
    // quartet), 9 DMAs a wave.
    auto row_src = [&](int idx_lane, int grp) -> const uint8_t* {
      const int row_idx = __shfl(idx_lane, KV_FP8 ? 16 * wave + (lane >> 2) : 16 * wave + 8 * grp + (lane >> 3));
      return gather_src<KV_FP8>(a, row_idx, valid_of(row_idx), lane);
    };
    auto issue_gather = [&](int idx_lane, int buf) {
      if (KV_FP8) {
        dma_quartets(row_src(idx_lane, 0),
                     __builtin_amdgcn_readfirstlane(tile_lds0 + buf * kCodeTileBytes + wave * 1024));
        return;
      }
#pragma unroll
      for (int grp = 0; grp < 2; ++grp)
        dma_octets(row_src(idx_lane, grp),
                   __builtin_amdgcn_readfirstlane(tile_lds0 + buf * kTileBytes + (2 * wave + grp) * 1024));
    };

    // per-lane LDS byte offsets of the operand reads (the tile layout above)
    const int sw_k = rsw(hl);
    const int kb0 = hl * 128 + ((G ^ sw_k) * 16);              // K chunk 4ks + G, ks even
    const int kb1 = hl * 128 + (((4 + G) ^ sw_k) * 16);        // ks odd
    const Fp8Offsets f8 = fp8_offsets(lane);                  // FP8 pool: K and V^T reads of the codes
    const int sw_v = rsw(4 * G + ((lane >> 2) & 3));
    const int vrow = (4 * G + ((lane >> 2) & 3)) * 128 + (lane & 1) * 8;
    const int vrow8 = f8.v[0] - G * 16;                         // FP8: the lane's V^T row offset
    // The wave's first column tile within its 64-column segment: 0, or 2 for the
    // odd waves when a wave owns 32 columns (four column parts).
    const int c0 = kWCols < 64 ? ((kWCols / 16) * wave) & 3 : 0;
    int vb[4], vb8[4];                                          // the wave's column tile ct & 3
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int cm = (c0 + m) & 3;
      vb[m] = vrow + (((2 * cm + ((lane & 3) >> 1)) ^ sw_v) * 16);
      vb8[m] = vrow8 + ((cm ^ G) * 16);
    }

    // ---- prologue: the head tile's 16 Q rows into LDS at kQOffset; wave w
    // stages rows [8 (w & 1), +8) (waves 2-3 repeat waves 0-1's rows, same
    // bytes, so every wave has the same loads in flight).
    int idx_cur;
    {
      const int r0 = 8 * (wave & 1) + (lane >> 3);
      const int chunk = ((lane & 7) ^ rsw(lane >> 3)) * 16;
      const uint8_t* qbase = (const uint8_t*)(q_ptr + ((int64_t)t * h_q + 16 * htile) * 576);
      idx_cur = load_idx_and_q1(idx_row + min(job.b0 * kBlk + lane, topk - 1), qbase + (int64_t)r0 * 1152 + chunk,
                                __builtin_amdgcn_readfirstlane(tile_lds0 + kQOffset + (wave & 1) * 1024));
    }

    auto run_pass = [&](const bool first) __attribute__((always_inline)) -> bool {
    bool overflow = false;
    if (!first) idx_cur = load_idx(job.b0);
    idx_cur = slot_in(job.b0) ? idx_cur : -1;
    issue_gather(idx_cur, 0);
    int idx_nxt = load_idx(job.b0 + 1);
    bool valid_cur = valid_of(idx_cur);
    if (first) {
      // Q rows landed (issued first; block b0's 18 DMAs (FP8: 9) and, with the
      // look-ahead, the next index load stay in flight).
      wait_q_rows<PREFETCH, KV_FP8 ? 9 : 18>();
      lds_barrier();
      load_q_frags(qf, lds_addr(s_tile) + kQOffset, kb0, kb1);
    }
    // FP8: block b0's row scales (stored at the top of the block loop).
    float sc_cur = (KV_FP8 && valid_cur) ? a.kv_scale[idx_cur] : 0.f;

    // One block a job and a bf16 pool: a wave scores the rows it gathered
    // itself, so QK^T waits for its own DMAs only, and the weight exchange's
    // barrier orders the other waves' rows before the V^T reads.
    constexpr bool kOwnRows = !PREFETCH && !KV_FP8;
    for (int b = job.b0; b < job.b1; ++b) {
      const int cur = (b - job.b0) & 1;
      wait_vmem_all();          // this wave's share of block b has landed
      if (KV_FP8 && wave == 0) s_scale[cur][lane] = sc_cur;
      if (kOwnRows)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      else
        lds_barrier();          // ... and every wave's; block b-1 and its weights fully consumed
      // slot s of the block is valid iff bit s is set (the same in every wave)
      const uint64_t vmask = __ballot(valid_cur);
      const uint32_t vquart = (uint32_t)(vmask >> (16 * wave));
      const bool blk_any = vmask != 0ull;

      // Block b+1: bf16, one DMA per QK^T k-step (group 0's 9, then group 1's);
      // FP8, one per k-step pair.  Masked rows and rows past the job's last
      // block copy the zero row.
      bool valid_nxt = false;
      float sc_nxt = 0.f;
      const uint8_t* gsrc0 = g_zero_row;
      const uint8_t* gsrc1 = g_zero_row;
      uint32_t gbase0 = 0u, gbase1 = 0u;
      if (PREFETCH) {
        idx_nxt = slot_in(b + 1) ? idx_nxt : -1;
        valid_nxt = valid_of(idx_nxt);
        if (KV_FP8 && wave == 0 && valid_nxt) sc_nxt = a.kv_scale[idx_nxt];
        gsrc0 = row_src(idx_nxt, 0);
        if (KV_FP8) {
          gbase0 = __builtin_amdgcn_readfirstlane(tile_lds0 + (cur ^ 1) * kCodeTileBytes + wave * 1024);
        } else {
          gsrc1 = row_src(idx_nxt, 1);
          gbase0 = __builtin_amdgcn_readfirstlane(tile_lds0 + (cur ^ 1) * kTileBytes + (2 * wave) * 1024);
          gbase1 = __builtin_amdgcn_readfirstlane(tile_lds0 + (cur ^ 1) * kTileBytes + (2 * wave + 1) * 1024);
        }
      }
      auto gather_dma = [&](const int d) __attribute__((always_inline)) {
        if (!PREFETCH) return;
        if (KV_FP8) {
          if ((d & 1) == 0) return;
          switch (d >> 1) {
            case 0: dma_one<4096, 64, 0>(gsrc0, gbase0); break;
            case 1: dma_one<4096, 64, 1>(gsrc0, gbase0); break;
            case 2: dma_one<4096, 64, 2>(gsrc0, gbase0); break;
            case 3: dma_one<4096, 64, 3>(gsrc0, gbase0); break;
            case 4: dma_one<4096, 64, 4>(gsrc0, gbase0); break;
            case 5: dma_one<4096, 64, 5>(gsrc0, gbase0); break;
            case 6: dma_one<4096, 64, 6>(gsrc0, gbase0); break;
            case 7: dma_one<4096, 64, 7>(gsrc0, gbase0); break;
            default: dma_one<4096, 64, 8>(gsrc0, gbase0); break;
          }
          return;
        }
        switch (d) {
          case 0: dma_one<8192, 128, 0>(gsrc0, gbase0); break;
          case 1: dma_one<8192, 128, 1>(gsrc0, gbase0); break;
          case 2: dma_one<8192, 128, 2>(gsrc0, gbase0); break;
          case 3: dma_one<8192, 128, 3>(gsrc0, gbase0); break;
          case 4: dma_one<8192, 128, 4>(gsrc0, gbase0); break;
          case 5: dma_one<8192, 128, 5>(gsrc0, gbase0); break;
          case 6: dma_one<8192, 128, 6>(gsrc0, gbase0); break;
          case 7: dma_one<8192, 128, 7>(gsrc0, gbase0); break;
          case 8: dma_one<8192, 128, 8>(gsrc0, gbase0); break;
          case 9: dma_one<8192, 128, 0>(gsrc1, gbase1); break;
          case 10: dma_one<8192, 128, 1>(gsrc1, gbase1); break;
          case 11: dma_one<8192, 128, 2>(gsrc1, gbase1); break;
          case 12: dma_one<8192, 128, 3>(gsrc1, gbase1); break;
          case 13: dma_one<8192, 128, 4>(gsrc1, gbase1); break;
          case 14: dma_one<8192, 128, 5>(gsrc1, gbase1); break;
          case 15: dma_one<8192, 128, 6>(gsrc1, gbase1); break;
          case 16: dma_one<8192, 128, 7>(gsrc1, gbase1); break;
          default: dma_one<8192, 128, 8>(gsrc1, gbase1); break;
        }
      };
      const int idx_after = load_idx(b + 2);

      // Block b's operands: bf16 rows, or the e4m3 codes converted in registers.
      const uint32_t tl = lds_addr(s_tile + cur * (KV_FP8 ? kCodeTileBytes : kTileBytes));
      uint32_t kbase[4], vbase[4];
      if constexpr (KV_FP8) {
        kbase[0] = opaque(tl + f8.k[0]);
        kbase[1] = opaque(tl + f8.k[1]);
        kbase[2] = kbase[3] = 0u;
        const uint32_t tlv = tl + ((kCols * cpart + kWCols * wave) / 64) * 4096;     // the 64-column segment of the wave's first column
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + vb8[m]);
      } else {
        kbase[0] = opaque(tl + kb0);
        kbase[1] = opaque(tl + kb1);
        kbase[2] = opaque(tl + kb0 + 65536);
        kbase[3] = opaque(tl + kb1 + 65536);
        const uint32_t tlv = tl + ((kCols * cpart + kWCols * wave) / 64) * 8192;
#pragma unroll
        for (int m = 0; m < 4; ++m) vbase[m] = opaque(tlv + vb[m]);
      }
      auto kfrag = [&](int ks, int st) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_kfrag(kbase[ks & 1] + (ks >> 1) * 4096 + st * 1024);
        const uint32_t kp = kbase[(ks & 1) + (ks >= 16 ? 2 : 0)] + ((ks >> 1) & 7) * 8192 + st * 2048;
        return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)kp;
      };
      auto vfrag = [&](int ct, int kk) -> bf16x8 {
        if constexpr (KV_FP8) return fp8_vfrag(vbase[ct & 3] + (ct >> 2) * 4096 + kk * 2048);
        const uint32_t vp = vbase[ct & 3] + (ct >> 2) * 8192 + kk * 4096;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)vp);
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)(vp + 2048));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
        return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
      };

      // ---- S^T = K . Q^T over this wave's slot tile: one accumulator
      constexpr int kAheadK = 3, kRing = kAheadK + 1, kAheadV = 4;
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        bf16x8 kf[kRing];
#pragma unroll
        for (int a0 = 0; a0 < kAheadK; ++a0) kf[a0] = kfrag(a0, wave);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if (ks + kAheadK < 18) kf[(ks + kAheadK) % kRing] = kfrag(ks + kAheadK, wave);
          __builtin_amdgcn_sched_barrier(0);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % kRing], qf[ks], sacc, 0, 0, 0);
          gather_dma(ks);               // the next block's DMAs 0..17, one per k-step
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax of this wave's 16 slots (lane: slots 16 wave + 4G + i)
      constexpr int kAV = kAheadV < 2 * kCt ? kAheadV : 2 * kCt;
      bf16x8 vf[kAV + 1];
      if (!kOwnRows) {
#pragma unroll
        for (int a0 = 0; a0 < kAV; ++a0) vf[a0] = vfrag(a0 % kCt, a0 / kCt);
      }
      const uint32_t vbits = vquart >> (4 * G);
      f32x4 rsc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (KV_FP8) rsc = *(const f32x4*)&s_scale[cur][16 * wave + 4 * G];
      float tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bias = ((vbits >> i) & 1u) ? 0.f : kMaskedScore;
        tv[i] = KV_FP8 ? fmaf(sacc[i] * scale_log2, rsc[i], bias) : fmaf(sacc[i], scale_log2, bias);
      }
      float m = fmaxf(fmaxf(tv[0], tv[1]), fmaxf(tv[2], tv[3]));
      m = rows_max(m);
      m_seen = fmaxf(m_seen, m);
      if (!framed && blk_any) {
        // first block with a valid slot: the frame is the floor of the largest
        // of the four quarters' maxima
        if (G == 0) pex_own[hl] = m;
        lds_barrier();
        M_run = floorf(fmaxf(fmaxf(pex_of(0)[hl], pex_of(1)[hl]), fmaxf(pex_of(2)[hl], pex_of(3)[hl])));
        framed = true;
        lds_barrier();          // every wave has read the maxima before the weights overwrite them
      }
      overflow |= m > M_run + kFrameSlack;
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float tt = tv[e];
        float p = __builtin_amdgcn_exp2f(tt - M_run);
        l_run += p;
        if (KV_FP8) p *= rsc[e];
        pv[e] = p;
      }
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t h2 = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
        ph[j] = h2;
        pl[j] = pack_bf16x2(pv[2 * j] - __uint_as_float(h2 << 16), pv[2 * j + 1] - __uint_as_float(h2 & 0xFFFF0000u));
      }
      *(u32x2*)(s_pex[wave] + 8 * lane) = u32x2{ph[0], ph[1]};
      *(u32x2*)(s_pex[wave] + 512 + 8 * lane) = u32x2{pl[0], pl[1]};
      lds_barrier();            // every wave's weights (and, one block a job, rows) are in LDS
      if (kOwnRows) {
#pragma unroll
        for (int a0 = 0; a0 < kAV; ++a0) vf[a0] = vfrag(a0 % kCt, a0 / kCt);
      }

      // ---- O^T += V^T . P^T over the block: k-step kk takes the weights of
      // quarters 2kk (the first 4 k-indices of each lane's group) and 2kk + 1.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2 h0 = *(const u32x2*)(s_pex[2 * kk] + 8 * lane);
        const u32x2 h1 = *(const u32x2*)(s_pex[2 * kk + 1] + 8 * lane);
        const u32x2 l0 = *(const u32x2*)(s_pex[2 * kk] + 512 + 8 * lane);
        const u32x2 l1 = *(const u32x2*)(s_pex[2 * kk + 1] + 512 + 8 * lane);
        const bf16x8 pfh = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
        const bf16x8 pfl = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          const int n = kCt * kk + ct;            // position in the fragment stream
          if (n + kAV < 2 * kCt) vf[(n + kAV) % (kAV + 1)] = vfrag((n + kAV) % kCt, (n + kAV) / kCt);
          __builtin_amdgcn_sched_barrier(0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n % (kAV + 1)], pfh, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n % (kAV + 1)], pfl, acc[ct], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      valid_cur = valid_nxt;
      sc_cur = sc_nxt;
      idx_nxt = idx_after;
    }
    wait_vmem_all();            // the last block's look-ahead gather lands before LDS is reused
    return overflow;
    };

    // End of a pass: every wave posts its largest score, its denominator and
    // its overflow flag; returns whether any wave of the workgroup overflowed.
    auto end_exchange = [&](const bool overflow) __attribute__((always_inline)) -> bool {
      const bool any_ov = post_pass<kWaves>(overflow, m_seen, l_run, pex_own, s_pex[0], 1024, hl, G, lane);
      // the same sum, in the same order, in each of the four waves
      l_tot = ((pex_of(0)[16 + hl] + pex_of(1)[16 + hl]) + pex_of(2)[16 + hl]) + pex_of(3)[16 + hl];
      return any_ov;
    };

    if (end_exchange(run_pass(true))) {
      // the frame of the largest score of the four quarters bounds every weight by 2
      const float ms = fmaxf(fmaxf(pex_of(0)[hl], pex_of(1)[hl]), fmaxf(pex_of(2)[hl], pex_of(3)[hl]));
      M_run = ms > kMaskedScore ? floorf(ms) : kNoFrame;
      framed = true;
      l_run = 0.f;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      end_exchange(run_pass(false));
    }
  }

  // ---- epilogue: l = the four quarters' denominators (one frame), O = acc / l
  const float l = l_tot;
  const bool any = l > 0.f;
  const float lse = any ? M_run + __builtin_amdgcn_logf(l) : kNegInf;
  float oscale = any ? 1.0f / l : 0.f;
  if (DIRECT && a.sink != nullptr && any) {
    const float z = a.sink[head] * kLog2e - lse;
    oscale = oscale / (1.0f + __builtin_amdgcn_exp2f(z));
  }
  const int64_t rowt = (DIRECT ? (int64_t)t * h_q : ((int64_t)job.s * s_q + t) * h_q) + 16 * htile;
  if (wave == 0 && G == 0 && cpart == 0) {       // every column part holds the same LSE
    if (!DIRECT)
      a.lse_accum[rowt + hl] = lse;
    else if (a.lse_out != nullptr)
      a.lse_out[rowt + hl] = lse;
  }

  // Staging (row = head of the tile, the tiles are free): wave w writes its 16
  // heads x kWCols columns; after the barrier wave w stores heads [4w, 4w + 4)
  // in whole pieces of the workgroup's kCols columns.
  {
    uint8_t* stg = s_tile + hl * kStagePitch + (kWCols * wave + 4 * G) * 4;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) *(f32x4*)(stg + 64 * ct) = acc[ct] * oscale;
  }
  lds_barrier();
  const uint8_t* st = s_tile + 4 * wave * kStagePitch;
  const int64_t row0 = rowt + 4 * wave;
  const int col0 = kCols * cpart;
  if (!DIRECT || a.out_dtype == kOutF32) {       // 1 KB per instruction
    float* dst = (DIRECT ? (float*)a.out : a.o_accum) + row0 * 512 + col0;
#pragma unroll
    for (int j = 0; j < 4 * kCols / 256; ++j) {
      const int f = 256 * j + 4 * lane;
      const int r = f / kCols, c = f % kCols;
      *(f32x4*)(dst + r * 512 + c) = *(const f32x4*)(st + r * kStagePitch + 4 * c);
    }
  } else {                                       // bf16 (a direct FP8 output never takes this kernel)
    constexpr int kLanesPerRow = kCols / 8, kRowsPer = 64 / kLanesPerRow;
    const int rr = lane / kLanesPerRow, cc = 8 * (lane % kLanesPerRow);
    uint16_t* dst = (uint16_t*)a.out + row0 * 512 + col0 + cc;
#pragma unroll
    for (int j = 0; j < 4 / kRowsPer; ++j) {
      const int r = kRowsPer * j + rr;
      const f32x4 v0 = *(const f32x4*)(st + r * kStagePitch + 4 * cc);
      const f32x4 v1 = *(const f32x4*)(st + r * kStagePitch + 4 * cc + 16);
      *(u32x4*)(dst + r * 512) = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                       pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
    }
  }
  // Split jobs of a decode with an FP8 output: seed the combine's amax and counters.
  if (!DIRECT && a.out_scale != nullptr && job.s == 0 && job.part == 0 && tid == 0)
    seed_fp8_combine(a.out_scale, a.out, t, h_q);
}

template <bool KV_FP8, bool DIRECT, bool PREFETCH, int CP>
__global__ __launch_bounds__(kThreads) void decode_kernel4t(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t job0, DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds4tBytes];
  decode4t_body<KV_FP8, DIRECT, PREFETCH, CP>(indices, q_ptr, num_splits, n_blocks, s_q, topk, h_q, job0, a,
                                              (int)blockIdx.x, smem);
}

// One launch for more jobs than compute units, with a short last round: its
// first n_head workgroups run decode_kernel8p's body over jobs [0, n_head),
// the rest the jobs from n_head on in two parts (decode8h_body's head halves).
// The tail's workgroups start as soon as compute units free up, with no kernel
// boundary in between.  n_head is a multiple of 8, so the tail keeps the XCD
// grouping of a job's parts.
template <bool KV_FP8, bool DIRECT, bool PREFETCH>
__global__ __launch_bounds__(kThreads8) void decode_kernel8m(
    const int32_t* __restrict__ indices, const uint16_t* __restrict__ q_ptr, int32_t num_splits, int32_t n_blocks,
    int32_t s_q, int32_t topk, int32_t h_q, int32_t n_head, DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds8pBytes];
  const int block = (int)blockIdx.x;
  static_assert(kLds8pBytes >= kLds8hBytes, "the mixed launch's LDS holds either body");
  if (block < n_head)
    decode8p_body<KV_FP8, DIRECT, PREFETCH>(indices, q_ptr, num_splits, n_blocks, s_q, topk, h_q, 0, a, block,
                                            smem);
  else
    decode8h_body<KV_FP8, DIRECT, PREFETCH>(indices, q_ptr, num_splits, n_blocks, s_q, topk, h_q, n_head, a,
                                            block - n_head, smem);
}

// ---------------------------------------------------------------------------
// Combine: O = sum_s 2^(LSE_s - M) O_s / sum_s 2^(LSE_s - M), then the sink and
// the cast.  One wave merges one (token, head) row: lane l owns columns
// [4l, 4l+4) and [256+4l, 256+4l+4); lane s also loads split s's LSE.  The
// partial rows of the first splits are requested together with the LSEs, so
// the row loads do not wait for the weights.
// ---------------------------------------------------------------------------

struct Merged {
  f32x4 lo, hi;                      // columns 4l.., 256+4l..
  float lse;
};

// kMergeChunk: partial rows in flight per lane.  PARTS: the row is merged by
// 1, 2 or 4 waves.  PARTS = 1: lane l owns columns 4l.. and 256 + 4l.. (lo,
// hi); PARTS = 2: columns col0 + 4l.. (lo); PARTS = 4: columns col0 + 2l,
// col0 + 2l + 1 (lo[0], lo[1]).  Each element sees the same operations either way.
template <int kMergeChunk, int PARTS = 1>
__device__ __forceinline__ Merged merge_head(const CombineArgs& a, int t, int h, int col0 = 0) {
  constexpr int NV = PARTS == 1 ? 2 : 1;               // 16-byte (or 8-byte) pieces per lane and split
  const int lane = threadIdx.x & 63;
  const int S = a.num_splits;
  const int64_t row = (int64_t)t * a.h_q + h;
  const int64_t ostride = (int64_t)a.s_q * a.h_q * 512;
  const int lane_off = col0 + (PARTS == 4 ? 2 : 4) * lane;     // the lane's columns within a row
  const float* op = a.o_accum + row * 512 + lane_off;
  const float* zp = (const float*)g_zero_row + lane_off;        // a zero row for the slots past S
  auto piece = [&](const float* src) -> f32x4 {
    if (PARTS == 4) {
      const f32x2 x = *(const f32x2*)src;
      return f32x4{x[0], x[1], 0.f, 0.f};
    }
    return *(const f32x4*)src;
  };
  const float ls = lane < S ? a.lse_accum[lane * (int64_t)a.s_q * a.h_q + row] : kNegInf;
  // Split slots past S load the zero row (a cache hit after the first
  // workgroup, and no second request for a line already in flight) so the
  // loads are unconditional and the LSE wait leaves them in flight; their
  // terms are skipped below.
  f32x4 v[kMergeChunk][NV];
#pragma unroll
  for (int c = 0; c < kMergeChunk; ++c) {
    const float* src = c < S ? op + c * ostride : zp;
    v[c][0] = piece(src);
    if (NV == 2) v[c][NV - 1] = *(const f32x4*)(src + 256);
  }
  const float M = wave_max(ls);
  const float wl = (M == kNegInf || ls == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ls - M);
  const float ws = wave_sum(wl);
  Merged m;
  const bool none = M == kNegInf;    // every split empty: O = 0, LSE = -inf
  m.lse = none ? kNegInf : M + __builtin_amdgcn_logf(ws);
  // Terms past S are dropped by a select, not a branch, so that the loads
  // above are used on every path and stay where they are issued.
  f32x4 lo = {-0.f, -0.f, -0.f, -0.f}, hi = lo;   // IEEE additive identity: keeps the sign of -0 terms
#pragma unroll
  for (int c = 0; c < kMergeChunk; ++c) {
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), c));
    const f32x4 l2 = lo + w * v[c][0];
    lo = c < S ? l2 : lo;
    if (NV == 2) {
      const f32x4 h2 = hi + w * v[c][NV - 1];
      hi = c < S ? h2 : hi;
    }
  }
  for (int s0 = kMergeChunk; s0 < S; s0 += kMergeChunk) {
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      const float* src = s0 + c < S ? op + (s0 + c) * ostride : zp;
      v[c][0] = piece(src);
      if (NV == 2) v[c][NV - 1] = *(const f32x4*)(src + 256);
    }
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), min(s0 + c, 63)));
      const f32x4 l2 = lo + w * v[c][0];
      lo = s0 + c < S ? l2 : lo;
      if (NV == 2) {
        const f32x4 h2 = hi + w * v[c][NV - 1];
        hi = s0 + c < S ? h2 : hi;
      }
    }
  }
  float f = 1.0f / ws;
  if (a.sink != nullptr) f = f / (1.0f + __builtin_amdgcn_exp2f(a.sink[h] * kLog2e - m.lse));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  m.lo = none ? zero : lo * f;
  m.hi = none ? zero : hi * f;
  return m;
}

// bf16 / fp32 output.  PARTS = 1: HPW whole (token, head) rows per workgroup,
// one wave per row.  PARTS = 2 or 4 (HPW = 1): one wave merges 1 / PARTS of a
// row (workgroup PARTS r + j: row r, columns (512 / PARTS) j ..), so that a few
// rows spread over more waves, each with fewer loads in flight.
// The fields the first loads need come as leading (SGPR-preloaded) arguments.
template <int HPW, int CHUNK, int PARTS = 1>
__global__ __launch_bounds__(64 * HPW) void combine_kernel(const float* __restrict__ o_accum,
                                                           const float* __restrict__ lse_accum, int32_t s_q,
                                                           int32_t h_q, int32_t num_splits, CombineArgs args) {
  CombineArgs a = args;
  a.o_accum = o_accum;
  a.lse_accum = lse_accum;
  a.s_q = s_q;
  a.h_q = h_q;
  a.num_splits = num_splits;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bpt = (a.h_q + HPW - 1) / HPW;
  const int rb = (int)blockIdx.x / PARTS;
  const int col0 = (512 / PARTS) * ((int)blockIdx.x % PARTS);
  const int t = rb / bpt;
  const int h = (rb - t * bpt) * HPW + wave;
  if (h >= a.h_q) return;
  const Merged m = merge_head<CHUNK, PARTS>(a, t, h, col0);
  const int64_t row = (int64_t)t * a.h_q + h;
  constexpr int kLaneCols = PARTS == 4 ? 2 : 4;
  if (a.out_dtype == kOutF32) {
    float* o = (float*)a.out + row * 512 + col0 + kLaneCols * lane;
    if (PARTS == 4)
      *(f32x2*)o = f32x2{m.lo[0], m.lo[1]};
    else
      *(f32x4*)o = m.lo;
    if (PARTS == 1) *(f32x4*)(o + 256) = m.hi;
  } else {
    uint16_t* o = (uint16_t*)a.out + row * 512 + col0 + kLaneCols * lane;
    if (PARTS == 4)
      *(uint32_t*)o = pack_bf16x2(m.lo[0], m.lo[1]);
    else
      *(u32x2*)o = u32x2{pack_bf16x2(m.lo[0], m.lo[1]), pack_bf16x2(m.lo[2], m.lo[3])};
    if (PARTS == 1) *(u32x2*)(o + 256) = u32x2{pack_bf16x2(m.hi[0], m.hi[1]), pack_bf16x2(m.hi[2], m.hi[3])};
  }
  if (a.lse_out != nullptr && lane == 0 && col0 == 0) a.lse_out[row] = m.lse;
}

// FP8 output.  The token's scale needs the amax over all of its heads, and
// no memory beyond the caller's buffers is used.  Before the combine, the
// attention kernel (or combine_fp8_init_kernel, for the standalone combine)
// seeds out_scale[t] = -0.0 ("not yet a scale") and zeroes the first 8 bytes
// of the token's output rows, which the combine then uses as two counters
// until it writes its codes there (fp8_sync_words).
//
// One launch (combine_fp8_kernel) when every workgroup of the launch can be
// resident at once (at most one per compute unit): each workgroup merges its
// rows, keeps them in registers, raises the token's amax word with an atomic
// max and counts itself in with an acquire-release increment.  The workgroup
// that counts last reads the final amax, stores the scale in out_scale[t];
// the others wait for it to appear there.  Then every workgroup encodes its
// rows.  Only atomics carry data between workgroups.
//
// Larger launches take two passes that merge the rows twice (no workgroup
// waits for another):
//   amax:   per workgroup the largest amax raises out_scale[t] to
//           0x80000000 | bits(amax) with an unsigned atomic max (the bits of
//           non-negative floats order like the floats);
//   encode: turns the value it reads in out_scale[t] into the scale (amax /
//           448, or 1 for a zero amax, when the sign bit is set; the scale
//           itself otherwise), writes the codes; the wave of head 0 stores
//           the scale.  Every wave derives the same scale from either form.

__global__ __launch_bounds__(256) void combine_fp8_init_kernel(CombineArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < a.s_q) seed_fp8_combine(a.out_scale, a.out, t, a.h_q);
}

__device__ __forceinline__ float abs_max4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// Wave u of a launch with PARTS waves per row merges part u % PARTS of row
// u / PARTS (PARTS = 1: the whole row).
struct RowPart {
  int t, h, col0;
};
template <int PARTS>
__device__ __forceinline__ RowPart row_part(const CombineArgs& a, int64_t u) {
  const int64_t r = u / PARTS;
  RowPart p;
  p.col0 = (512 / PARTS) * (int)(u - r * PARTS);
  p.t = (int)(r / a.h_q);
  p.h = (int)(r - (int64_t)p.t * a.h_q);
  return p;
}

// e4m3 codes of a merged part row under the token's scale.
template <int PARTS>
__device__ __forceinline__ void store_codes(const CombineArgs& a, const RowPart& p, const Merged& m, float qscale) {
  const int lane = threadIdx.x & 63;
  uint8_t* orow = (uint8_t*)a.out + ((int64_t)p.t * a.h_q + p.h) * 512 + p.col0;
  if (PARTS == 4) {                        // columns col0 + 2l, col0 + 2l + 1
    const uint32_t w2 = e4m3_encode(m.lo[0] / qscale) | (e4m3_encode(m.lo[1] / qscale) << 8);
    *(uint16_t*)(orow + 2 * lane) = (uint16_t)w2;
  } else {
    uint32_t wlo = 0, whi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wlo |= e4m3_encode(m.lo[e] / qscale) << (8 * e);
      if (PARTS == 1) whi |= e4m3_encode(m.hi[e] / qscale) << (8 * e);
    }
    *(uint32_t*)(orow + 4 * lane) = wlo;
    if (PARTS == 1) *(uint32_t*)(orow + 256 + 4 * lane) = whi;
  }
}

// Polls a waiting workgroup makes for its token's scale before it gives up and
// takes NaN (only reachable if the token's workgroups were not all resident).
constexpr int kScaleSpinLimit = 1 << 16;

// One-launch FP8 combine: HW waves per workgroup, PARTS waves per row; a
// token's h_q * PARTS waves fill h_q * PARTS / HW whole workgroups.
template <int HW, int CHUNK, int PARTS>
__global__ __launch_bounds__(64 * HW) void combine_fp8_kernel(CombineArgs a) {
  static_assert(HW == 4 || HW == 8 || HW == 16, "waves per workgroup");
  __shared__ float s_amax[HW];
  __shared__ float s_scale;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowPart p = row_part<PARTS>(a, (int64_t)blockIdx.x * HW + wave);
  const Merged m = merge_head<CHUNK, PARTS>(a, p.t, p.h, p.col0);
  if (lane == 0 && p.col0 == 0 && a.lse_out != nullptr) a.lse_out[(int64_t)p.t * a.h_q + p.h] = m.lse;
  const float amax_w = wave_max(PARTS == 1 ? fmaxf(abs_max4(m.lo), abs_max4(m.hi)) : abs_max4(m.lo));
  if (lane == 0) s_amax[wave] = amax_w;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < HW; ++w) v = fmaxf(v, s_amax[w]);
    uint32_t* sync = fp8_sync_words(a.out, p.t, a.h_q);
    uint32_t* scale_word = (uint32_t*)a.out_scale + p.t;
    const uint32_t n_wg = (uint32_t)(a.h_q * PARTS / HW);
    __hip_atomic_fetch_max(sync + 1, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Release: this workgroup's amax is in before its count.  The last one to
    // count in then acquires, so it sees every amax (an acquire in every
    // workgroup measured 1.2 us slower at 16 tokens: each invalidates its L2).
    const uint32_t before = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    float sc;
    if (before == n_wg - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const float amax = __uint_as_float(__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      sc = amax > 0.f ? amax / 448.0f : 1.0f;
      __hip_atomic_store(scale_word, __float_as_uint(sc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t bits = 0x80000000u;
      for (int n = 0; n < kScaleSpinLimit && bits == 0x80000000u; ++n) {
        __builtin_amdgcn_s_sleep(1);
        bits = __hip_atomic_load(scale_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      sc = bits == 0x80000000u ? __builtin_nanf("") : __uint_as_float(bits);
    }
    s_scale = sc;
  }
  __syncthreads();
  store_codes<PARTS>(a, p, m, s_scale);
}

// Two-pass FP8 combine, amax pass: HW waves per workgroup, whose amaxes meet
// in LDS, so a token sees fewer atomics.  PARTS = 1: one wave per (token,
// head) row, HW = 16 keeping the atomics of a large batch few.
template <int HW, int CHUNK, int PARTS>
__global__ __launch_bounds__(64 * HW) void combine_fp8_amax_kernel(CombineArgs a) {
  __shared__ float s_amax[HW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowPart p = row_part<PARTS>(a, (int64_t)blockIdx.x * HW + wave);
  const Merged m = merge_head<CHUNK, PARTS>(a, p.t, p.h, p.col0);
  const float amax = wave_max(PARTS == 1 ? fmaxf(abs_max4(m.lo), abs_max4(m.hi)) : abs_max4(m.lo));
  if (lane == 0 && p.col0 == 0 && a.lse_out != nullptr) a.lse_out[(int64_t)p.t * a.h_q + p.h] = m.lse;
  if (lane == 0) s_amax[wave] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < HW; ++w) v = fmaxf(v, s_amax[w]);
    __hip_atomic_fetch_max((uint32_t*)a.out_scale + p.t, 0x80000000u | __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Two-pass FP8 combine, encode pass: HPW whole rows per workgroup, merged again.
template <int HPW, int CHUNK>
__global__ __launch_bounds__(64 * HPW) void combine_fp8_encode_kernel(CombineArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowPart p = row_part<1>(a, (int64_t)blockIdx.x * HPW + wave);
  const Merged m = merge_head<CHUNK, 1>(a, p.t, p.h, 0);
  const uint32_t v = __hip_atomic_load((const uint32_t*)a.out_scale + p.t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float qscale;
  if (v & 0x80000000u) {
    const float amax = __uint_as_float(v & 0x7FFFFFFFu);
    qscale = amax > 0.f ? amax / 448.0f : 1.0f;
  } else {
    qscale = __uint_as_float(v);
  }
  store_codes<1>(a, p, m, qscale);
  if (p.h == 0 && lane == 0) a.out_scale[p.t] = qscale;
}

}  // namespace

namespace {
// One launch over jobs [job0, job1) with cs column parts.
template <bool DIRECT, bool PREFETCH>
hipError_t launch_jobs(const DecodeArgs& a, bool kv_fp8, int cs, int job0, int job1, hipStream_t stream) {
  const unsigned n_jobs = (unsigned)(job1 - job0);
  const dim3 grid(cs == 1 ? n_jobs : (n_jobs + 7) / 8 * 8 * cs);
  const int tiles = a.h_q / 16;
  const bool fp8_direct = DIRECT && a.out_dtype == kOutFp8;
  // 64 heads in one column part, or a direct FP8 output (one part; fewer
  // heads are padded to 64): the 8-wave kernel whose wave pairs trade their
  // weights.
  if (cs == 1 && (a.h_q == 64 || fp8_direct)) {
    if (kv_fp8)
      hipLaunchKernelGGL((decode_kernel8p<true, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                         a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, job0, a);
    else
      hipLaunchKernelGGL((decode_kernel8p<false, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                         a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, job0, a);
    return hipGetLastError();
  }
  // 64 heads in two parts: head halves that do not repeat QK^T.
  if (a.h_q == 64 && cs == 2) {
    if (kv_fp8)
      hipLaunchKernelGGL((decode_kernel8h<true, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                         a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, job0, a);
    else
      hipLaunchKernelGGL((decode_kernel8h<false, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                         a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, job0, a);
    return hipGetLastError();
  }
  // One 16-head tile per 4-wave workgroup, whole or in 2 or 4 column parts
  // (64 heads: 4, 8 or 16 workgroups a job; 32: 2, 4 or 8; 16: 1, 2 or 4),
  // none repeating another tile's QK^T.
  if (!fp8_direct && cs >= tiles && cs <= 4 * tiles && (a.h_q < 64 || cs >= 4)) {
#define SMLA_LAUNCH_4T(FP8, CPV)                                                                             \
  hipLaunchKernelGGL((decode_kernel4t<FP8, DIRECT, PREFETCH, CPV>), grid, dim3(kThreads), 0, stream, a.indices, \
                     a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, job0, a)
    const int cp = cs / tiles;
    if (kv_fp8 && cp == 1)
      SMLA_LAUNCH_4T(true, 1);
    else if (kv_fp8 && cp == 2)
      SMLA_LAUNCH_4T(true, 2);
    else if (kv_fp8)
      SMLA_LAUNCH_4T(true, 4);
    else if (cp == 1)
      SMLA_LAUNCH_4T(false, 1);
    else if (cp == 2)
      SMLA_LAUNCH_4T(false, 2);
    else
      SMLA_LAUNCH_4T(false, 4);
#undef SMLA_LAUNCH_4T
    return hipGetLastError();
  }
  return hipErrorInvalidValue;                  // no other part count is planned
}

// The whole launch plan.  With one column part and more jobs than compute
// units, the last round would leave CUs idle: when it holds at most half of
// them, its jobs take 2, 4 or 8 parts (the largest that keeps it within one
// round; 4 at most for 16 heads), so it finishes sooner -- in the same launch
// for 64 heads (decode_kernel8m), else in a second one.  A
// direct FP8 output keeps one part (its scale needs every column).
template <bool DIRECT, bool PREFETCH>
hipError_t launch_decode_cs(const DecodeArgs& a, bool kv_fp8, hipStream_t stream) {
  const int n_jobs = a.s_q * (DIRECT ? 1 : a.num_splits);
  const int cus = a.cus;
  const int tail = cus > 0 ? n_jobs % cus : 0;
  if (a.col_parts == 1 && n_jobs > cus && tail > 0 && 2 * tail <= cus && !(DIRECT && a.out_dtype == kOutFp8)) {
    const int cs_tail = min(8 * tail <= cus ? 8 : 4 * tail <= cus ? 4 : 2, 4 * (a.h_q / 16));
    const int n_head = n_jobs - tail;
    if (a.h_q == 64 && n_head % 8 == 0) {     // both bodies in one launch, the tail in 2 parts
      const dim3 grid((unsigned)(n_head + (tail + 7) / 8 * 8 * 2));
      if (kv_fp8)
        hipLaunchKernelGGL((decode_kernel8m<true, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                           a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, n_head, a);
      else
        hipLaunchKernelGGL((decode_kernel8m<false, DIRECT, PREFETCH>), grid, dim3(kThreads8), 0, stream, a.indices,
                           a.q, a.num_splits, a.n_blocks, a.s_q, a.topk, a.h_q, n_head, a);
      return hipGetLastError();
    }
    const hipError_t e = launch_jobs<DIRECT, PREFETCH>(a, kv_fp8, 1, 0, n_jobs - tail, stream);
    if (e != hipSuccess) return e;
    return launch_jobs<DIRECT, PREFETCH>(a, kv_fp8, cs_tail, n_jobs - tail, n_jobs, stream);
  }
  return launch_jobs<DIRECT, PREFETCH>(a, kv_fp8, a.col_parts, 0, n_jobs, stream);
}
}  // namespace

// Jobs of one block at most (num_splits >= block count) need no look-ahead.
hipError_t launch_decode_partial(const DecodeArgs& a, bool kv_fp8, hipStream_t stream) {
  return a.num_splits >= a.n_blocks ? launch_decode_cs<false, false>(a, kv_fp8, stream)
                                    : launch_decode_cs<false, true>(a, kv_fp8, stream);
}

hipError_t launch_decode_direct(const DecodeArgs& a, bool kv_fp8, hipStream_t stream) {
  return launch_decode_cs<true, true>(a, kv_fp8, stream);
}

namespace {
// The FP8 output's combine.  One launch while the whole grid fits one
// workgroup per compute unit: quarter rows per wave, 2 rows a workgroup, up to
// as many rows as CUs; half rows, 2 rows a workgroup, up to twice as many;
// half rows, 8 a workgroup, up to 4x; then whole rows, 8 or 16 a workgroup.
// A token's workgroups all count in on one counter, so fewer workgroups a
// token mean fewer atomics in line there: 2 rows a workgroup at one token
// (32 workgroups) measured 0.6 us faster than 1 (64), and 8 at 16 tokens 2 us
// faster than 4.  Else the two passes.
template <int CHUNK>
void launch_combine_fp8(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.s_q * a.h_q;
  const int64_t cus = a.cus;
  const dim3 g4((unsigned)(rows / 4)), g8((unsigned)(rows / 8)), g16((unsigned)(rows / 16));
  if (rows <= cus)
    hipLaunchKernelGGL((combine_fp8_kernel<8, CHUNK, 4>), dim3((unsigned)(rows / 2)), dim3(512), 0, stream, a);
  else if (rows <= 2 * cus)
    hipLaunchKernelGGL((combine_fp8_kernel<4, CHUNK, 2>), dim3((unsigned)(rows / 2)), dim3(256), 0, stream, a);
  else if (rows <= 4 * cus)
    hipLaunchKernelGGL((combine_fp8_kernel<16, CHUNK, 2>), dim3((unsigned)(rows / 8)), dim3(1024), 0, stream, a);
  else if (rows <= 8 * cus)
    hipLaunchKernelGGL((combine_fp8_kernel<8, CHUNK, 1>), g8, dim3(512), 0, stream, a);
  else if (rows <= 16 * cus)
    hipLaunchKernelGGL((combine_fp8_kernel<16, CHUNK, 1>), g16, dim3(1024), 0, stream, a);
  else {
    hipLaunchKernelGGL((combine_fp8_amax_kernel<16, CHUNK, 1>), g16, dim3(1024), 0, stream, a);
    hipLaunchKernelGGL((combine_fp8_encode_kernel<4, CHUNK>), g4, dim3(256), 0, stream, a);
  }
}

// CHUNK: partial rows requested per pass (4, 8, 12 or 16), the smallest that
// holds every split, so few loads repeat a row needlessly.
template <int CHUNK>
hipError_t launch_combine_chunk(const CombineArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.s_q * a.h_q);
  const unsigned blocks4 = (unsigned)(a.s_q * ((a.h_q + 3) / 4));
  if (a.out_dtype == kOutFp8) {
    if (!a.scale_ready)
      hipLaunchKernelGGL(combine_fp8_init_kernel, dim3((unsigned)((a.s_q + 255) / 256)), dim3(256), 0, stream, a);
    launch_combine_fp8<CHUNK>(a, stream);
  } else if (a.heads_per_wg == -1) {              // a quarter of a row per wave
    hipLaunchKernelGGL((combine_kernel<1, CHUNK, 4>), dim3(4 * rows), dim3(64), 0, stream, a.o_accum,
                       a.lse_accum, a.s_q, a.h_q, a.num_splits, a);
  } else if (a.heads_per_wg == 0) {               // half a row per wave
    hipLaunchKernelGGL((combine_kernel<1, CHUNK, 2>), dim3(2 * rows), dim3(64), 0, stream, a.o_accum,
                       a.lse_accum, a.s_q, a.h_q, a.num_splits, a);
  } else {
    hipLaunchKernelGGL((combine_kernel<4, CHUNK>), dim3(blocks4), dim3(256), 0, stream, a.o_accum, a.lse_accum,
                       a.s_q, a.h_q, a.num_splits, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  static std::atomic<void*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.num_splits <= 4) return launch_combine_chunk<4>(a, stream);
  if (a.num_splits == 5) return launch_combine_chunk<5>(a, stream);
  if (a.num_splits == 6) return launch_combine_chunk<6>(a, stream);
  if (a.num_splits <= 8) return launch_combine_chunk<8>(a, stream);
  if (a.num_splits <= 10) return launch_combine_chunk<10>(a, stream);
  if (a.num_splits <= 12) return launch_combine_chunk<12>(a, stream);
  return launch_combine_chunk<16>(a, stream);
}

}  // namespace smla
