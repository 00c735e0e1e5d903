/*
 * smla.h -- C ABI of the split-KV sparse MLA decode library for MI355X (gfx950).
 *
 * The operation (FlashMLA PR #25, "Purpose" and "What changes"; "The Split-K
 * Dispatch", "The LSE Combine Strategy"; cudnn-frontend PR #768, commit
 * messages):
 *
 *   For every query token t and head h, over the valid slots i of the token's
 *   top-k index list (slot valid iff 0 <= indices[t][i] < n_pool):
 *     s_i      = softmax_scale * <q[t][h][0:576], kv[indices[t][i]][0:576]>
 *     O[t][h]  = sum_i softmax(s)_i * kv[indices[t][i]][0:512]
 *     LSE[t][h]= log2(sum_i exp(s_i))                      (log2 units)
 *   The slot list is cut into blocks of `split_block` slots and the blocks
 *   into `num_splits` near-equal consecutive ranges, the remainder going to
 *   the leading splits (a split past the end is empty).  Each (token, split)
 *   job writes its own partial O normalised by its own softmax denominator and
 *   its own LSE; an empty or fully masked split writes O = +0.0, LSE = -inf.
 *   The combine merges the splits: M = max_s LSE_s, w_s = 2^(LSE_s - M),
 *   O = sum_s w_s O_s / sum_s w_s, LSE = M + log2(sum_s w_s); it then folds
 *   in the optional per-head sink logit (natural-log units, one extra key with
 *   a zero value row: O *= 1 / (1 + exp(sink[h] - LSE*ln2))) and casts.  The
 *   returned LSE never includes the sink.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, never synchronises, and enqueues its kernels on
 *     `stream` (a hipStream_t; NULL = the null stream), so calls can be
 *     captured into a HIP graph.
 *   - Optional pointers are NULL when absent.
 *   - Errors are returned as an smla_status before anything is enqueued; a
 *     kernel-launch failure is reported as SMLA_ERR_HIP.  No call aborts.
 *   - Index contents are not checked on the host: out-of-range values are
 *     masked on the device and never dereferenced.
 *   - All layouts are dense, row-major, in the shapes given below; there are
 *     no caller strides except kv_row_stride.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARG = 1,        /* NULL required pointer, non-positive size, bad enum */
  SMLA_ERR_UNSUPPORTED = 2,        /* h_q not in {16, 32, 64}, split_block != 64, too large */
  SMLA_ERR_MISSING_WORKSPACE = 3,  /* num_splits > 1 without o_accum and lse_accum */
  SMLA_ERR_MISALIGNED = 4,         /* a pointer or the row stride breaks 16-byte alignment */
  SMLA_ERR_HIP = 5,                /* the HIP runtime rejected a launch */
  SMLA_ERR_SCRATCH_TOO_SMALL = 6   /* sparse_mla_decode_noalloc: the partials exceed its scratch */
} smla_status;

typedef enum { SMLA_KV_BF16 = 0, SMLA_KV_FP8_E4M3 = 1 } smla_kv_dtype;
typedef enum { SMLA_OUT_BF16 = 0, SMLA_OUT_FP32 = 1, SMLA_OUT_FP8_E4M3 = 2 } smla_out_dtype;

#define SMLA_D_QK 576          /* 512 latent + 64 RoPE dimensions per KV row */
#define SMLA_D_V 512           /* the value is the first 512 dimensions of the row */
#define SMLA_SPLIT_BLOCK 64    /* slots per KV block, the unit of the split partition */
#define SMLA_MAX_SPLITS 64
/* Bytes of device scratch (one copy per GPU) that hold the split partials of
 * sparse_mla_decode_noalloc. */
#define SMLA_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef struct {
  int32_t s_q;             /* query tokens, >= 1 */
  int32_t h_q;             /* query heads per token: 16, 32 or 64 */
  int32_t topk;            /* index slots per token, >= 1 */
  int32_t split_block;     /* slots per KV block; must be SMLA_SPLIT_BLOCK */
  int64_t n_pool;          /* rows in the KV pool, >= 1 */
  int64_t kv_row_stride;   /* elements between consecutive pool rows (bf16: elements,
                              FP8: bytes); >= 576 and a multiple of 16 bytes */
  float softmax_scale;     /* multiplies q.k (e.g. 1/sqrt(576)) */
  int32_t kv_dtype;        /* smla_kv_dtype */
  int32_t out_dtype;       /* smla_out_dtype */
} smla_params;

/*
 * sparse_mla_decode -- the decode step: per-(token, split) attention jobs and,
 * when an output is requested, the combine.  The jobs, the block ranges and the
 * partials follow FlashMLA PR #25, "What changes" (each (token, split) job walks
 * its own KV block range and stores an fp32 O normalised by its own denominator
 * plus a log2-space LSE, no cast); the empty split and the remainder rule follow
 * cudnn-frontend PR #768, commit messages; the direct path is FlashMLA PR #25's
 * unsplit path, whose epilogue casts ("What changes", last item).  With an FP8
 * output the combine owns the amax of the recombined output (cudnn-frontend PR
 * #768, commit messages).
 *
 *   q          [s_q][h_q][576] bf16, 16-byte aligned.
 *   kv_pool    [n_pool][kv_row_stride]: bf16 (SMLA_KV_BF16) or e4m3fn codes
 *              (SMLA_KV_FP8_E4M3); only the first 576 entries of a row are read.
 *   kv_scale   [n_pool] f32 per-row dequantisation scale (FP8 pool only, else NULL):
 *              row value = e4m3(code) * kv_scale[row].
 *   indices    [s_q][topk] int32 pool rows; values outside [0, n_pool) are masked.
 *   num_splits 1 .. SMLA_MAX_SPLITS (more splits than blocks is allowed: the
 *              trailing splits are empty).  smla_choose_num_splits() gives a
 *              default for the shape.
 *   sink       [h_q] f32 per-head sink logit, or NULL for none.
 *   o_accum    [num_splits][s_q][h_q][512] f32 partial outputs, split-major,
 *              16-byte aligned, or NULL.
 *   lse_accum  [num_splits][s_q][h_q] f32 partial log2 LSEs, or NULL.
 *   out        [s_q][h_q][512] in out_dtype (bf16 / f32 / e4m3fn codes), 16-byte
 *              aligned, or NULL.
 *   out_scale  [s_q] f32 per-token dequantisation scale of an FP8 output
 *              (amax over the token's h_q*512 outputs / 448, or 1 when that amax
 *              is 0); required when out_dtype is FP8 and out is given, else unused.
 *   lse_out    [s_q][h_q] f32 final log2 LSE (without the sink), or NULL.
 *
 * Modes:
 *   - o_accum and lse_accum NULL, num_splits == 1: direct path.  One job per
 *     token computes the final output with the sink and the cast fused into its
 *     epilogue.  `out` is required.
 *   - o_accum and lse_accum given: every job writes its partials (the FlashMLA
 *     partial protocol); if `out` is given the combine runs after it on the same
 *     stream, otherwise the caller combines (combine_splits).  On return
 *     o_accum and lse_accum hold the partials in either case, so the caller may
 *     combine them again.
 *   - num_splits > 1 with either accumulator NULL: SMLA_ERR_MISSING_WORKSPACE.
 *   - Giving only one of o_accum / lse_accum: SMLA_ERR_MISSING_WORKSPACE.
 * An FP8 `out` of the split mode doubles as the combine's counters while the
 * call runs (the first 8 bytes of each token's rows), until the codes land.
 */
smla_status sparse_mla_decode(const smla_params* p, const void* q, const void* kv_pool,
                              const float* kv_scale, const int32_t* indices, int32_t num_splits,
                              const float* sink, float* o_accum, float* lse_accum, void* out,
                              float* out_scale, float* lse_out, void* stream);

/*
 * sparse_mla_decode_noalloc -- sparse_mla_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split partials live in a scratch array
 * of the library, SMLA_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends.  Same arguments and results as sparse_mla_decode without o_accum and
 * lse_accum; `out` is required.  num_splits == 1 takes the direct path (no
 * scratch); num_splits > 1 needs smla_partial_bytes(s_q, h_q, num_splits) plus
 * at most 255 bytes of alignment within the scratch, else the call returns
 * SMLA_ERR_SCRATCH_TOO_SMALL before anything is enqueued.
 * The call allocates nothing: its first call on a device looks the scratch's
 * address up (hipGetSymbolAddress) and keeps it for that device.  Every call
 * on one GPU uses that GPU's one scratch, which keeps the last call's
 * partials: calls ordered on one stream are safe, calls that overlap on one
 * GPU (other streams, concurrent graph replays) race.  Nothing in it needs to
 * start at zero: every job writes its partials before the combine reads them.
 */
smla_status sparse_mla_decode_noalloc(const smla_params* p, const void* q, const void* kv_pool,
                                      const float* kv_scale, const int32_t* indices, int32_t num_splits,
                                      const float* sink, void* out, float* out_scale, float* lse_out,
                                      void* stream);

/*
 * combine_splits -- merge split partials (as written by sparse_mla_decode) into
 * the final output ("The Split-K Dispatch", "The LSE Combine Strategy": weights
 * 2^(LSE_s - max LSE); FlashMLA PR #25, "What changes": the combine applies the
 * sink, once).  Same shapes and meaning as above; o_accum, lse_accum and out
 * are required and o_accum / lse_accum are only read; p->kv_dtype, topk,
 * n_pool, kv_row_stride and softmax_scale are not used.  A split whose LSE is
 * -inf contributes nothing; a (token, head) with every split at -inf gets
 * O = 0 and LSE = -inf.
 */
smla_status combine_splits(const smla_params* p, int32_t num_splits, const float* o_accum,
                           const float* lse_accum, const float* sink, void* out,
                           float* out_scale, float* lse_out, void* stream);

/*
 * smla_choose_num_splits -- a split count for the shape that gives small decode
 * batches enough (token, split) jobs to fill `num_cus` compute units and keeps
 * large batches unsplit ("The Split-K Dispatch", "The Reasoning Behind the
 * Design", "Adaptive NSPLIT": the split count adapts to the batch).  With
 * x = num_cus / s_q compute units per token: S = x / 8 (rounded down) when
 * x >= 40, 4 when x >= 16, 2 when x >= 8, else 1, capped at the block count
 * (and SMLA_MAX_SPLITS).  Jobs then run as up to 16 workgroups each (one per
 * part of the heads and of the output columns).
 * Deterministic in its arguments, so a captured graph stays valid.  Returns
 * >= 1, or 0 when an argument is non-positive.
 */
int32_t smla_choose_num_splits(int32_t s_q, int32_t h_q, int32_t topk, int32_t num_cus);

/*
 * smla_partial_bytes -- bytes of o_accum plus lse_accum for the shape:
 * num_splits * s_q * h_q * (512 * 4 + 4) (FlashMLA PR #25, "Measured", gives
 * the o_accum part).  Returns 0 when an argument is non-positive.
 */
size_t smla_partial_bytes(int32_t s_q, int32_t h_q, int32_t num_splits);

/*
 * smla_validate -- the host-side argument check sparse_mla_decode performs,
 * without launching anything (the host rules of FlashMLA PR #25, "Limitations /
 * follow-ups": partial buffers only where supported; cudnn-frontend PR #768,
 * commit messages: a split needs its LSE workspace and takes no caller stride).  Pointers are only tested for NULL and
 * alignment, never dereferenced, so host addresses may stand in for them.
 */
smla_status smla_validate(const smla_params* p, const void* q, const void* kv_pool,
                          const float* kv_scale, const int32_t* indices, int32_t num_splits,
                          const float* o_accum, const float* lse_accum, const void* out,
                          const float* out_scale);

/*
 * ---------------------------------------------------------------------------
 * Split-KV FP8 prefill attention (cudnn-frontend PR #768, "split kv ports":
 * the split-KV port of an FP8 SDPA prefill kernel with head dimension 128).
 *
 *   For batch b, query row i < seqlen_q[b] and query head h, over the keys
 *   j < seqlen_kv[b] that the row may see (all of them, or, with `causal`,
 *   j <= i + seqlen_kv[b] - seqlen_q[b]: the mask aligned to the bottom-right
 *   corner), with KV head h / (h_q / h_kv):
 *     s_ij = softmax_scale * <q_i, k_j>,  O_i = sum_j softmax(s)_ij v_j,
 *     LSE_i = ln sum_j exp(s_ij)                          (natural log)
 *   Q, K and V are e4m3fn codes times one float32 descale factor per tensor.
 *   Under a split, each tile of q_tile query rows takes its masked KV range
 *   (the keys its last row may see) in blocks of kv_block keys, cut into
 *   split_kv near-equal chunks with the remainder on the leading chunks; every
 *   row still applies its own mask inside its chunk.  A split writes its
 *   partial O (normalised by its own denominator) and its LSE into split-major
 *   slots; an empty chunk writes O = +0, LSE = -inf.  The combine merges the
 *   splits (weights exp(LSE_s - max LSE)), applies the sink once (one extra key
 *   of logit sink[h], natural-log units, with a zero value row), casts, and
 *   owns the amax of the recombined output.  The returned LSE excludes the
 *   sink.  A row that sees no key gets O = 0 and LSE = -inf.
 * ---------------------------------------------------------------------------
 */
typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t h_q;             /* query heads, a multiple of h_kv, <= 256 */
  int32_t h_kv;            /* KV heads >= 1 */
  int32_t head_dim;        /* must be 128 */
  int32_t max_s_q;         /* padded query rows per batch (Sq), >= 1 */
  int32_t max_s_kv;        /* padded keys per batch (Skv), >= 1 */
  int32_t causal;          /* 1: bottom-right causal mask, 0: none */
  int32_t q_tile;          /* query rows per tile; must be 64 */
  int32_t kv_block;        /* keys per KV block; must be 64 */
  float softmax_scale;     /* multiplies q.k (e.g. 1/sqrt(128)) */
  float descale_q, descale_k, descale_v;   /* per-tensor dequantisation factors */
  int32_t out_dtype;       /* SMLA_OUT_BF16 or SMLA_OUT_FP32 */
} smla_prefill_params;

/*
 * sdpa_fp8_prefill -- split-KV FP8 prefill attention and, when an output is
 * requested, its combine.
 *
 *   q          [B][Sq][h_q][128] e4m3fn codes, 16-byte aligned.
 *   k, v       [B][Skv][h_kv][128] e4m3fn codes, 16-byte aligned.
 *   seqlen_q   [B] int32 device array: query rows present (values are clamped
 *              into [0, Sq] on the device).
 *   seqlen_kv  [B] int32 device array: keys present (clamped into [0, Skv]).
 *   split_kv   1 .. SMLA_MAX_SPLITS.  smla_prefill_choose_splits() gives a
 *              default for the shape.
 *   sink       [h_q] f32 per-head sink logit, or NULL.
 *   o_part     [split_kv][B][Sq][h_q][128] f32 split partials, 16-byte aligned,
 *              or NULL; lse_part [split_kv][B][Sq][h_q] f32, or NULL.
 *   out        [B][Sq][h_q][128] bf16 or f32 (out_dtype), 16-byte aligned, or
 *              NULL (partial-only); rows i >= seqlen_q[b] are not written.
 *   lse_out    [B][Sq][h_q] f32 final natural-log LSE (without the sink), or NULL.
 *   amax_out   one f32: max |O| over the written rows, before the cast, or NULL.
 * Modes as sparse_mla_decode: no partials and split_kv == 1 is the direct path
 * (one kernel writes O, the sink and the amax fused in its epilogue); with
 * partials every split writes them and, if `out` is given, the combine runs;
 * split_kv > 1 without partials is SMLA_ERR_MISSING_WORKSPACE.  The score
 * scale softmax_scale * descale_q * descale_k must be positive and at least
 * 2^-100 (in float32, times log2 e), else SMLA_ERR_INVALID_ARG.
 */
smla_status sdpa_fp8_prefill(const smla_prefill_params* p, const void* q, const void* k, const void* v,
                             const int32_t* seqlen_q, const int32_t* seqlen_kv, int32_t split_kv,
                             const float* sink, float* o_part, float* lse_part, void* out, float* lse_out,
                             float* amax_out, void* stream);

/*
 * smla_prefill_partial_bytes -- bytes of o_part plus lse_part:
 * split_kv * batch * max_s_q * h_q * (128 * 4 + 4); 0 for a non-positive argument.
 */
size_t smla_prefill_partial_bytes(int32_t batch, int32_t max_s_q, int32_t h_q, int32_t split_kv);

/*
 * smla_prefill_choose_splits -- a split count that gives a grid of few query
 * tiles enough workgroups for `num_cus` compute units (a performance choice,
 * cudnn-frontend PR #768 leaves SPLIT_KV to the caller).  The unsplit launch
 * has batch * ceil(max_s_q / 64) * h_q / HPW workgroups, HPW = 2 query heads a
 * workgroup when h_q / h_kv is even, else 1: 1 when that fills two rounds
 * (two workgroups a compute unit), else the count that brings it to about two
 * rounds, capped at the KV blocks of the longest range (ceil(max_s_kv / 64))
 * and at 16.  Deterministic.  Returns >= 1, or 0 for a non-positive argument
 * or h_q not a multiple of h_kv.
 */
int32_t smla_prefill_choose_splits(int32_t batch, int32_t max_s_q, int32_t max_s_kv, int32_t h_q, int32_t h_kv,
                                   int32_t num_cus);

/* smla_status_string -- a static, human-readable name of a status code. */
const char* smla_status_string(smla_status s);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
