// C ABI of the split-KV sparse MLA decode library: argument checks, the split
// count heuristic and the launch sequence.  The kernels live in
// smla_kernels.hip.  Nothing here allocates memory or synchronises.

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "smla.h"
#include "smla_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t n_blocks_of(int32_t topk) { return (topk + SMLA_SPLIT_BLOCK - 1) / SMLA_SPLIT_BLOCK; }

// Compute units of the current device (cached per device; 256 if unknown).
int32_t device_cus() {
  static std::atomic<int32_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Checks shared by both entry points: the shape fields that the combine uses.
smla_status check_common_shape(const smla_params* p, int32_t num_splits) {
  if (p == nullptr) return SMLA_ERR_INVALID_ARG;
  if (p->s_q < 1 || p->s_q > (1 << 22)) return p->s_q < 1 ? SMLA_ERR_INVALID_ARG : SMLA_ERR_UNSUPPORTED;
  if (p->h_q != 16 && p->h_q != 32 && p->h_q != 64) return SMLA_ERR_UNSUPPORTED;
  if (num_splits < 1) return SMLA_ERR_INVALID_ARG;
  if (num_splits > SMLA_MAX_SPLITS) return SMLA_ERR_UNSUPPORTED;
  if ((int64_t)p->s_q * num_splits > INT32_MAX) return SMLA_ERR_UNSUPPORTED;
  if (p->out_dtype != SMLA_OUT_BF16 && p->out_dtype != SMLA_OUT_FP32 && p->out_dtype != SMLA_OUT_FP8_E4M3)
    return SMLA_ERR_INVALID_ARG;
  return SMLA_OK;
}

}  // namespace

extern "C" {

const char* smla_status_string(smla_status s) {
  switch (s) {
    case SMLA_OK: return "SMLA_OK";
    case SMLA_ERR_INVALID_ARG: return "SMLA_ERR_INVALID_ARG";
    case SMLA_ERR_UNSUPPORTED: return "SMLA_ERR_UNSUPPORTED";
    case SMLA_ERR_MISSING_WORKSPACE: return "SMLA_ERR_MISSING_WORKSPACE";
    case SMLA_ERR_MISALIGNED: return "SMLA_ERR_MISALIGNED";
    case SMLA_ERR_HIP: return "SMLA_ERR_HIP";
    case SMLA_ERR_SCRATCH_TOO_SMALL: return "SMLA_ERR_SCRATCH_TOO_SMALL";
  }
  return "SMLA_ERR_UNKNOWN";
}

size_t smla_partial_bytes(int32_t s_q, int32_t h_q, int32_t num_splits) {
  if (s_q < 1 || h_q < 1 || num_splits < 1) return 0;
  return (size_t)num_splits * (size_t)s_q * (size_t)h_q * (size_t)(SMLA_D_V * 4 + 4);
}

int32_t smla_choose_num_splits(int32_t s_q, int32_t h_q, int32_t topk, int32_t num_cus) {
  if (s_q < 1 || h_q < 1 || topk < 1 || num_cus < 1) return 0;
  const int32_t n_blk = n_blocks_of(topk);
  // By compute units per token x = num_cus / s_q: S = x / 8 when x >= 40, 4
  // when x >= 16, 2 when x >= 8, else 1 (capped at the block count).  Jobs
  // then run as 2, 4 or 8 workgroups, each owning part of the heads or of the
  // output columns (sparse_mla_decode picks the most that fit one round over
  // the CUs).  This was the best measured S at every batch size of a sweep on
  // a 256-CU MI355X (s_q = 1 ... 128, within 2% at s_q = 24): more splits
  // shorten a small batch's critical path, but every split adds a partial to
  // write and merge.
  const int64_t cus = num_cus, t = s_q;
  int32_t s = cus >= 40 * t ? (int32_t)(cus / (8 * t)) : cus >= 16 * t ? 4 : cus >= 8 * t ? 2 : 1;
  const int32_t cap = n_blk < SMLA_MAX_SPLITS ? n_blk : SMLA_MAX_SPLITS;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

smla_status smla_validate(const smla_params* p, const void* q, const void* kv_pool, const float* kv_scale,
                          const int32_t* indices, int32_t num_splits, const float* o_accum,
                          const float* lse_accum, const void* out, const float* out_scale) {
  smla_status st = check_common_shape(p, num_splits);
  if (st != SMLA_OK) return st;
  if (p->topk < 1 || p->n_pool < 1) return SMLA_ERR_INVALID_ARG;
  if (p->split_block != SMLA_SPLIT_BLOCK) return SMLA_ERR_UNSUPPORTED;
  if (p->kv_dtype != SMLA_KV_BF16 && p->kv_dtype != SMLA_KV_FP8_E4M3) return SMLA_ERR_INVALID_ARG;
  if (!isfinite(p->softmax_scale)) return SMLA_ERR_INVALID_ARG;
  if (p->kv_row_stride < SMLA_D_QK) return SMLA_ERR_INVALID_ARG;
  const int64_t elem = p->kv_dtype == SMLA_KV_BF16 ? 2 : 1;
  if (p->kv_row_stride > (INT64_MAX / 4) / elem) return SMLA_ERR_UNSUPPORTED;
  if ((p->kv_row_stride * elem) % 16 != 0) return SMLA_ERR_MISALIGNED;
  if (q == nullptr || kv_pool == nullptr || indices == nullptr) return SMLA_ERR_INVALID_ARG;
  if (p->kv_dtype == SMLA_KV_FP8_E4M3 && kv_scale == nullptr) return SMLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_pool)) return SMLA_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(indices) & 3u) != 0) return SMLA_ERR_MISALIGNED;
  if (kv_scale != nullptr && (reinterpret_cast<uintptr_t>(kv_scale) & 3u) != 0) return SMLA_ERR_MISALIGNED;
  const bool has_o = o_accum != nullptr, has_l = lse_accum != nullptr;
  if (has_o != has_l) return SMLA_ERR_MISSING_WORKSPACE;
  if (num_splits > 1 && !has_o) return SMLA_ERR_MISSING_WORKSPACE;
  if (!has_o && out == nullptr) return SMLA_ERR_INVALID_ARG;     // direct path needs an output
  if (has_o && !aligned16(o_accum)) return SMLA_ERR_MISALIGNED;
  if (has_l && (reinterpret_cast<uintptr_t>(lse_accum) & 3u) != 0) return SMLA_ERR_MISALIGNED;
  if (out != nullptr) {
    if (!aligned16(out)) return SMLA_ERR_MISALIGNED;
    if (p->out_dtype == SMLA_OUT_FP8_E4M3 && out_scale == nullptr) return SMLA_ERR_INVALID_ARG;
  }
  return SMLA_OK;
}

}  // extern "C"

namespace {

// The combine launch sequence; scale_ready: an FP8 output's out_scale and
// token counters already hold the combine's starting values (seeded by the
// attention kernel).
smla_status run_combine(const smla_params* p, int32_t num_splits, const float* o_accum, const float* lse_accum,
                        const float* sink, void* out, float* out_scale, float* lse_out, void* stream,
                        bool scale_ready) {
  smla_status st = check_common_shape(p, num_splits);
  if (st != SMLA_OK) return st;
  if (o_accum == nullptr || lse_accum == nullptr) return SMLA_ERR_MISSING_WORKSPACE;
  if (out == nullptr) return SMLA_ERR_INVALID_ARG;
  if (p->out_dtype == SMLA_OUT_FP8_E4M3 && out_scale == nullptr) return SMLA_ERR_INVALID_ARG;
  if (!aligned16(o_accum) || !aligned16(out)) return SMLA_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(lse_accum) & 3u) != 0) return SMLA_ERR_MISALIGNED;
  smla::CombineArgs a;
  a.o_accum = o_accum;
  a.lse_accum = lse_accum;
  a.sink = sink;
  a.out = out;
  a.out_scale = out_scale;
  a.lse_out = lse_out;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.num_splits = num_splits;
  a.out_dtype = p->out_dtype;
  // A few rows spread over more waves, each merging part of a row (fewer loads
  // in flight per wave): a quarter of a row per wave while four times the rows
  // fit the CUs, half a row up to twice as many rows as CUs (measured on the
  // MI355X: 2.9 -> 2.2 us at one token, 2.5 -> 2.3 us at 4 to 6), then four
  // whole rows per workgroup.
  const int64_t rows = (int64_t)p->s_q * p->h_q;
  const int32_t cus = device_cus();
  a.heads_per_wg = 4 * rows <= cus ? -1 : rows <= 2 * cus ? 0 : 4;
  a.scale_ready = scale_ready ? 1 : 0;
  a.cus = cus;
  return smla::launch_combine(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

}  // namespace

extern "C" {

smla_status combine_splits(const smla_params* p, int32_t num_splits, const float* o_accum,
                           const float* lse_accum, const float* sink, void* out, float* out_scale,
                           float* lse_out, void* stream) {
  return run_combine(p, num_splits, o_accum, lse_accum, sink, out, out_scale, lse_out, stream, false);
}

smla_status sparse_mla_decode(const smla_params* p, const void* q, const void* kv_pool, const float* kv_scale,
                              const int32_t* indices, int32_t num_splits, const float* sink, float* o_accum,
                              float* lse_accum, void* out, float* out_scale, float* lse_out, void* stream) {
  smla_status st = smla_validate(p, q, kv_pool, kv_scale, indices, num_splits, o_accum, lse_accum, out, out_scale);
  if (st != SMLA_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fp8 = p->kv_dtype == SMLA_KV_FP8_E4M3;
  smla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_pool);
  a.kv_scale = kv_scale;
  a.indices = indices;
  a.sink = sink;
  a.o_accum = o_accum;
  a.lse_accum = lse_accum;
  a.out = out;
  const bool direct = o_accum == nullptr;
  // split mode with an FP8 output to follow: the attention kernel seeds out_scale and the token counters
  const bool seed_scale = !direct && out != nullptr && p->out_dtype == SMLA_OUT_FP8_E4M3;
  a.out_scale = (direct || seed_scale) ? out_scale : nullptr;
  a.lse_out = lse_out;
  a.n_pool = p->n_pool;
  a.row_stride_bytes = p->kv_row_stride * (fp8 ? 1 : 2);
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.topk = p->topk;
  a.num_splits = num_splits;
  a.n_blocks = n_blocks_of(p->topk);
  a.out_dtype = p->out_dtype;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  // Few jobs leave most compute units idle: then several workgroups share each
  // job, each owning part of its heads and of its 512 output columns.  64
  // heads: 1 to 16 workgroups a job; fewer heads: one per 16-head tile, times
  // 1, 2 or 4 column parts.  Not for a direct FP8 output, whose scale needs
  // every head and column of a token.
  const int64_t jobs = (int64_t)p->s_q * (direct ? 1 : num_splits);
  const int32_t cus = device_cus();
  const int32_t tiles = p->h_q / 16;
  if (direct && p->out_dtype == SMLA_OUT_FP8_E4M3)
    a.col_parts = 1;
  else if (p->h_q == 64)
    a.col_parts = 16 * jobs <= cus ? 16 : 8 * jobs <= cus ? 8 : 4 * jobs <= cus ? 4 : 2 * jobs <= cus ? 2 : 1;
  else
    a.col_parts = 4 * tiles * jobs <= cus ? 4 * tiles : 2 * tiles * jobs <= cus ? 2 * tiles : tiles;
  a.cus = cus;

  if (direct) {        // direct path: one job per token, fused epilogue
    return smla::launch_decode_direct(a, fp8, hs) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
  }
  if (smla::launch_decode_partial(a, fp8, hs) != hipSuccess) return SMLA_ERR_HIP;
  if (out == nullptr) return SMLA_OK;   // partial-only: the caller combines
  return run_combine(p, num_splits, o_accum, lse_accum, sink, out, out_scale, lse_out, stream, seed_scale);
}

smla_status sparse_mla_decode_noalloc(const smla_params* p, const void* q, const void* kv_pool,
                                      const float* kv_scale, const int32_t* indices, int32_t num_splits,
                                      const float* sink, void* out, float* out_scale, float* lse_out,
                                      void* stream) {
  if (out == nullptr) return SMLA_ERR_INVALID_ARG;
  if (num_splits == 1)       // the direct path has no partials
    return sparse_mla_decode(p, q, kv_pool, kv_scale, indices, 1, sink, nullptr, nullptr, out, out_scale, lse_out,
                             stream);
  const smla_status st = check_common_shape(p, num_splits);
  if (st != SMLA_OK) return st;
  // o_accum at the start of the scratch, lse_accum after it on a 256-byte boundary
  const size_t rows = (size_t)num_splits * (size_t)p->s_q * (size_t)p->h_q;
  const size_t lse_off = (rows * SMLA_D_V * 4 + 255) & ~(size_t)255;
  if (lse_off + rows * 4 > SMLA_NOALLOC_SCRATCH_BYTES) return SMLA_ERR_SCRATCH_TOO_SMALL;
  void* base = nullptr;
  if (smla::noalloc_scratch(&base) != hipSuccess) return SMLA_ERR_HIP;
  return sparse_mla_decode(p, q, kv_pool, kv_scale, indices, num_splits, sink, static_cast<float*>(base),
                           reinterpret_cast<float*>(static_cast<uint8_t*>(base) + lse_off), out, out_scale, lse_out,
                           stream);
}

size_t smla_prefill_partial_bytes(int32_t batch, int32_t max_s_q, int32_t h_q, int32_t split_kv) {
  if (batch < 1 || max_s_q < 1 || h_q < 1 || split_kv < 1) return 0;
  return (size_t)split_kv * (size_t)batch * (size_t)max_s_q * (size_t)h_q * (size_t)(128 * 4 + 4);
}

int32_t smla_prefill_choose_splits(int32_t batch, int32_t max_s_q, int32_t max_s_kv, int32_t h_q, int32_t h_kv,
                                   int32_t num_cus) {
  if (batch < 1 || max_s_q < 1 || max_s_kv < 1 || h_q < 1 || h_kv < 1 || num_cus < 1 || h_q % h_kv != 0) return 0;
  // Workgroups of the unsplit launch: one per (batch, 64-row tile, head pair
  // when a KV head serves an even number of query heads, else head).
  const int64_t hpw = (h_q / h_kv) % 2 == 0 ? 2 : 1;
  const int64_t tiles = (int64_t)batch * ((max_s_q + 63) / 64) * (h_q / hpw);
  const int64_t target = 2 * (int64_t)num_cus;
  if (tiles >= target) return 1;
  int64_t s = (target + tiles - 1) / tiles;
  const int64_t blocks = (max_s_kv + 63) / 64;
  if (s > blocks) s = blocks;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int32_t)s;
}

smla_status sdpa_fp8_prefill(const smla_prefill_params* p, const void* q, const void* k, const void* v,
                             const int32_t* seqlen_q, const int32_t* seqlen_kv, int32_t split_kv,
                             const float* sink, float* o_part, float* lse_part, void* out, float* lse_out,
                             float* amax_out, void* stream) {
  if (p == nullptr) return SMLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->h_q < 1 || p->h_kv < 1 || p->max_s_q < 1 || p->max_s_kv < 1) return SMLA_ERR_INVALID_ARG;
  if (p->head_dim != 128 || p->q_tile != 64 || p->kv_block != 64) return SMLA_ERR_UNSUPPORTED;
  if (p->h_q % p->h_kv != 0 || p->h_q > 256) return SMLA_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return SMLA_ERR_INVALID_ARG;
  if (p->out_dtype != SMLA_OUT_BF16 && p->out_dtype != SMLA_OUT_FP32) return SMLA_ERR_UNSUPPORTED;
  if (split_kv < 1) return SMLA_ERR_INVALID_ARG;
  if (split_kv > SMLA_MAX_SPLITS) return SMLA_ERR_UNSUPPORTED;
  if (!isfinite(p->softmax_scale) || !isfinite(p->descale_q) || !isfinite(p->descale_k) ||
      !isfinite(p->descale_v))
    return SMLA_ERR_INVALID_ARG;
  // the score scale in log2 units: the kernel needs it positive and not tiny
  const float scale_log2 = p->softmax_scale * p->descale_q * p->descale_k * 1.4426950408889634f;
  if (!(scale_log2 >= 0x1p-100f) || !isfinite(scale_log2)) return SMLA_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || seqlen_q == nullptr || seqlen_kv == nullptr)
    return SMLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return SMLA_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(seqlen_q) & 3u) != 0 || (reinterpret_cast<uintptr_t>(seqlen_kv) & 3u) != 0)
    return SMLA_ERR_MISALIGNED;
  const bool has_o = o_part != nullptr, has_l = lse_part != nullptr;
  if (has_o != has_l) return SMLA_ERR_MISSING_WORKSPACE;
  if (split_kv > 1 && !has_o) return SMLA_ERR_MISSING_WORKSPACE;
  if (!has_o && out == nullptr) return SMLA_ERR_INVALID_ARG;       // the direct path needs an output
  if (has_o && !aligned16(o_part)) return SMLA_ERR_MISALIGNED;
  if (has_l && (reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0) return SMLA_ERR_MISALIGNED;
  if (out != nullptr && !aligned16(out)) return SMLA_ERR_MISALIGNED;
  const int64_t n_tiles = (p->max_s_q + 63) / 64;
  const int64_t n_work = (int64_t)p->batch * split_kv * n_tiles * p->h_q;
  const int64_t rows = (int64_t)p->batch * p->max_s_q * p->h_q;
  if (n_work > INT32_MAX - 8 || (int64_t)p->batch * p->max_s_q > INT32_MAX ||
      (int64_t)p->batch * p->max_s_kv > INT32_MAX || rows * split_kv > ((int64_t)1 << 40))
    return SMLA_ERR_UNSUPPORTED;
  smla::PrefillArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.seqlen_q = seqlen_q;
  a.seqlen_kv = seqlen_kv;
  a.sink = sink;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.out = out;
  a.lse_out = lse_out;
  a.amax_out = out != nullptr ? amax_out : nullptr;    // partial-only: no output, no amax
  a.batch = p->batch;
  a.h_q = p->h_q;
  a.h_kv = p->h_kv;
  a.sq_max = p->max_s_q;
  a.skv_max = p->max_s_kv;
  a.num_splits = split_kv;
  a.n_tiles = (int32_t)n_tiles;
  a.causal = p->causal;
  a.out_dtype = p->out_dtype;
  a.scale_log2 = scale_log2;
  a.descale_v = p->descale_v;
  a.n_work = (int32_t)n_work;
  a.cus = device_cus();
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!has_o) return smla::launch_prefill(a, false, hs) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
  if (smla::launch_prefill(a, true, hs) != hipSuccess) return SMLA_ERR_HIP;
  if (out == nullptr) return SMLA_OK;
  return smla::launch_prefill_combine(a, hs) == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

}  // extern "C"
