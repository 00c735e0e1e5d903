"""Float64 CPU oracle for split-KV sparse MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
(to check one small GPU run) and by the ``cpu_baseline`` leg of ``bench.py``.
It shares no code with the HIP library and imports nothing from the package.

What is computed (sources are the three pages the method is described on):

* FlashMLA PR #25, "Purpose" and "What changes": every query token attends over
  its own top-k list of rows of a latent KV cache; the rows are shared by all
  query heads; the work is cut into (query token, KV split) jobs, each walking
  its own range of KV blocks; a job writes an fp32 output normalised by its own
  softmax denominator plus a log2-space log-sum-exp; a combine merges the
  splits and owns the attention sink.
* "The Split-K Dispatch" blog post, "The LSE Combine Strategy": the combine
  takes the maximum over the splits' log-sum-exps and weights each split by
  exp2 of its distance to that maximum.
* cudnn-frontend PR #768, commit messages: a split's KV range is a near-equal
  chunk with the remainder going to the leading splits; a chunk past the end
  is empty and enters the combine as O = 0, LSE = -inf; under a split the
  combine owns the FP8 amax of the recombined output.

Everything here is plain float64 numpy, written from the mathematical
definition (a softmax-weighted average of the gathered value rows), so that it
can be checked by eye.  Every function states the reading it takes where the
pages leave a step open.

Shapes (all arrays are numpy):
  q        [s_q, h_q, d_qk]   query, any float dtype (bf16 values held in f32 are exact)
  kv       [n_pool, d_qk]     latent KV pool (dequantised for the FP8 pool)
  indices  [s_q, topk]        int, -1 (or any value outside [0, n_pool)) = masked slot
  sink     [h_q] or None      per-head attention-sink logit, natural-log units
Outputs: O [s_q, h_q, d_v] float64, LSE [s_q, h_q] float64 in log2 units.
"""

import math

import numpy as np

D_QK = 576          # 512 latent + 64 RoPE dimensions per KV row
D_V = 512           # the value is the first 512 dimensions of the same row
LN2 = math.log(2.0)


# ----------------------------------------------------------------------------
# Index handling
# ----------------------------------------------------------------------------
def valid_mask(indices, n_pool):
    """True where a slot names a pool row.

    Reading: the pages only say that padded slots are masked (the workloads pad
    with -1); any value outside [0, n_pool) is treated like -1, i.e. it is
    never dereferenced and contributes nothing.
    """
    idx = np.asarray(indices)
    return (idx >= 0) & (idx < n_pool)


# ----------------------------------------------------------------------------
# Split partition (FlashMLA PR #25 "What changes": each job walks its own KV
# block range; cudnn-frontend PR #768: near-equal chunks, remainder to the
# leading splits, a chunk past the end is empty)
# ----------------------------------------------------------------------------
def split_block_ranges(n_blocks, num_splits):
    """Half-open block ranges [b0, b1) of every split, in split order.

    ``n_blocks`` blocks are cut into ``num_splits`` near-equal consecutive
    chunks; the first ``n_blocks % num_splits`` chunks get one block more.
    With more splits than blocks the trailing splits get empty ranges.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    base, rem = divmod(n_blocks, num_splits)
    ranges = []
    start = 0
    for s in range(num_splits):
        length = base + (1 if s < rem else 0)
        ranges.append((start, start + length))
        start += length
    assert start == n_blocks
    return ranges


def split_slot_ranges(topk, split_block, num_splits):
    """Slot-position ranges [i0, i1) of every split.

    Reading: the pages never name the size of a "KV block"; it is a parameter
    here (64 slots in every workload).  Blocks cover slot positions
    [b*split_block, (b+1)*split_block) clipped to topk; the last block may be
    ragged.
    """
    n_blocks = -(-topk // split_block)
    out = []
    for b0, b1 in split_block_ranges(n_blocks, num_splits):
        out.append((min(b0 * split_block, topk), min(b1 * split_block, topk)))
    return out


# ----------------------------------------------------------------------------
# Attention over one token's gathered rows (the plain definition)
# ----------------------------------------------------------------------------
def attend_token(q_t, kv, idx_t, n_pool, scale):
    """Softmax attention of all heads of one token over its valid slots.

    q_t [h_q, d_qk], idx_t [k].  Scores s_hi = scale * <q_h, K_i> over all 576
    dimensions; weights softmax_i(s_hi); output sum_i w_hi * K_i[:512];
    LSE_h = log2(sum_i exp(s_hi)).  No valid slot: O = 0, LSE = -inf.
    Returns (O [h_q, d_v], LSE [h_q]).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    h_q = q_t.shape[0]
    idx_t = np.asarray(idx_t)
    rows = idx_t[valid_mask(idx_t, n_pool)]
    if rows.size == 0:
        return np.zeros((h_q, D_V)), np.full(h_q, -np.inf)
    K = np.asarray(kv[rows], dtype=np.float64)              # [k, d_qk]
    s = float(scale) * (q_t @ K.T)                          # [h_q, k]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ K[:, :D_V]) / l
    lse = (m[:, 0] + np.log(l[:, 0])) / LN2
    return O, lse


def attend(q, kv, indices, n_pool, scale):
    """Final O and LSE of every (token, head), without any sink."""
    q = np.asarray(q)
    s_q, h_q = q.shape[0], q.shape[1]
    O = np.zeros((s_q, h_q, D_V))
    L = np.zeros((s_q, h_q))
    for t in range(s_q):
        O[t], L[t] = attend_token(q[t], kv, indices[t], n_pool, scale)
    return O, L


# ----------------------------------------------------------------------------
# Per-split partials (FlashMLA PR #25 "What changes": a partial normalised by
# the split's own denominator plus a log2-space LSE; cudnn-frontend PR #768:
# an empty split is O = 0, LSE = -inf)
# ----------------------------------------------------------------------------
def split_partials(q, kv, indices, n_pool, scale, num_splits, split_block=64):
    """o_accum [S, s_q, h_q, d_v] and lse_accum [S, s_q, h_q], split-major.

    Split s of token t is the plain attention of that token restricted to the
    slot positions of split s; a split with no valid slot is (0, -inf).
    """
    q = np.asarray(q)
    indices = np.asarray(indices)
    s_q, h_q = q.shape[0], q.shape[1]
    topk = indices.shape[1]
    o_acc = np.zeros((num_splits, s_q, h_q, D_V))
    lse_acc = np.full((num_splits, s_q, h_q), -np.inf)
    for s, (i0, i1) in enumerate(split_slot_ranges(topk, split_block, num_splits)):
        for t in range(s_q):
            o_acc[s, t], lse_acc[s, t] = attend_token(q[t], kv, indices[t, i0:i1], n_pool, scale)
    return o_acc, lse_acc


# ----------------------------------------------------------------------------
# Combine ("The Split-K Dispatch", "The LSE Combine Strategy"; FlashMLA PR #25)
# ----------------------------------------------------------------------------
def combine_partials(o_acc, lse_acc):
    """Merge split partials with the log-sum-exp rule.

    For every (token, head): M = max_s LSE_s; w_s = 2^(LSE_s - M);
    O = sum_s w_s O_s / sum_s w_s; LSE = M + log2(sum_s w_s).  Every split at
    -inf (no valid slot anywhere): O = 0, LSE = -inf.
    """
    o_acc = np.asarray(o_acc, dtype=np.float64)
    lse_acc = np.asarray(lse_acc, dtype=np.float64)
    M = lse_acc.max(axis=0)                                       # [s_q, h_q]
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(lse_acc), 0.0, np.exp2(lse_acc - M_safe[None]))
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    O = (w[..., None] * o_acc).sum(axis=0) / wsum_safe[..., None]
    O[empty] = 0.0
    lse = np.where(empty, -np.inf, M_safe + np.log2(wsum_safe))
    return O, lse


def apply_sink(O, lse, sink):
    """Fold a per-head sink logit into the normalised output.

    Readings (the pages only say the combine applies the sink, once):
    the sink acts as one extra key per head whose logit is ``sink[h]`` in
    natural-log units (not multiplied by the softmax scale) and whose value
    row is zero.  Then O' = sum_i e^{s_i} v_i / (sum_i e^{s_i} + e^{sink}),
    i.e. O' = O * 1 / (1 + exp(sink - LSE*ln2)).  The LSE is returned without
    the sink.  No valid slot (LSE = -inf) leaves O = 0.
    """
    if sink is None:
        return np.array(O, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    with np.errstate(over="ignore"):
        z = sink[None, :] - lse * LN2                       # [s_q, h_q]
        factor = 1.0 / (1.0 + np.exp(z))
    factor = np.where(np.isneginf(lse), 0.0, factor)
    return O * factor[..., None]


def decode(q, kv, indices, n_pool, scale, sink=None):
    """Final (O with sink, LSE without sink) by the plain definition."""
    O, lse = attend(q, kv, indices, n_pool, scale)
    return apply_sink(O, lse, sink), lse


def decode_split(q, kv, indices, n_pool, scale, num_splits, split_block=64, sink=None):
    """Same result through partials and the combine (split + combine path)."""
    o_acc, lse_acc = split_partials(q, kv, indices, n_pool, scale, num_splits, split_block)
    O, lse = combine_partials(o_acc, lse_acc)
    return apply_sink(O, lse, sink), lse


# ----------------------------------------------------------------------------
# FP8 e4m3 (OCP "e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits, no infinities, S.1111.111 is NaN, largest finite 448)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of every e4m3fn code as float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x):
    """Round-to-nearest-even e4m3fn code of each value, saturating at +-448.

    The rounding is exact: it is decided on the float64 value handed in (the
    caller chooses in which precision that value was formed).  The sign bit
    follows the sign of x, -0.0 and values that round to zero included.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: value = m * 2^-9, m in 0..7; m = 8 is the smallest normal (code 8)
    sub = a < 2.0 ** -6
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normal range: a = f * 2^E with f in [1, 2)
    fr, ex = np.frexp(np.where(sub, 1.0, a))               # a = fr * 2^ex, fr in [0.5, 1)
    E = ex - 1
    mant = np.rint((fr * 2.0 - 1.0) * 8.0).astype(np.int64)   # 0..8, ties to even
    carry = mant == 8
    E = np.where(carry, E + 1, E)
    mant = np.where(carry, 0, mant)
    normal_code = ((E + 7) << 3) | mant
    normal_code = np.minimum(normal_code, 0x7E)                # 448 saturates (0x7E)
    code = np.where(sub, code, normal_code)
    return (code | sign).astype(np.uint8)


def fp8_quantize_per_token(O):
    """Per-token FP8 output: scale = amax/448 (1.0 when amax is 0), codes of O/scale.

    Reading: the pages say the combine owns the amax of the recombined output
    (cudnn-frontend PR #768); the scale convention (one fp32 scale per query
    token over all heads and the 512 value dimensions, amax/448) is a choice
    this oracle fixes.  Decided in float64.
    """
    O = np.asarray(O, dtype=np.float64)
    amax = np.abs(O).reshape(O.shape[0], -1).max(axis=1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    codes = e4m3_encode(O / scale[:, None, None])
    return codes, scale


def fp8_quantize_per_token_f32(O32):
    """The same quantisation decided in float32, as a float32 kernel takes it.

    amax is exact in float32; scale = fl32(amax / 448); each code is the RNE
    e4m3 code of fl32(O / scale) (IEEE float32 division).
    """
    O32 = np.asarray(O32, dtype=np.float32)
    amax = np.abs(O32).reshape(O32.shape[0], -1).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    ratio = (O32 / scale[:, None, None]).astype(np.float32)
    return e4m3_encode(ratio.astype(np.float64)), scale


def dequantize_fp8_rows(codes, row_scale):
    """FP8 KV pool rows to float64: value(code) * row_scale[row]."""
    return e4m3_decode(codes) * np.asarray(row_scale, dtype=np.float64)[:, None]


def gather_dequantize_fp8(codes, row_scale, rows):
    """Dequantise only the named pool rows (keeps a large pool out of float64)."""
    rows = np.asarray(rows)
    return e4m3_decode(codes[rows]) * np.asarray(row_scale, dtype=np.float64)[rows][:, None]


class Fp8Pool:
    """Row-indexable view of an FP8 pool that dequantises on access.

    ``Fp8Pool(codes, scale)[rows]`` returns float64 rows, so every function
    above accepts it in place of a float KV pool.
    """

    def __init__(self, codes, row_scale):
        self.codes = codes
        self.row_scale = row_scale

    def __getitem__(self, rows):
        return gather_dequantize_fp8(self.codes, self.row_scale, rows)


def partial_bytes(s_q, h_q, num_splits, d_v=D_V):
    """Bytes of the fp32 partial outputs (FlashMLA PR #25 "Measured"):
    num_splits * s_q * h_q * d_v * 4, plus 4 bytes of LSE per (split, token, head)."""
    return num_splits * s_q * h_q * (d_v * 4 + 4)
