"""Float64 CPU oracle for split-KV FP8 prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/`` and by the ``cpu_baseline`` leg of
``bench.py``.  It shares no code with the HIP library and imports nothing from
the package.

What is computed (cudnn-frontend PR #768, "split kv ports", its commit
messages and reviews, which describe the split-KV port of an FP8 prefill SDPA
kernel with head dimension 128):

* Every query row of a batch attends, per query head, over the keys its mask
  allows (the "already-masked KV range"); several query heads share one KV
  head ("qh_per_kh"); every batch has its own key count ("seqlen_kv").
* Under a split, each tile of query rows takes its masked KV range, cut into
  SPLIT_KV near-equal chunks of KV blocks with the remainder on the leading
  chunks; a chunk past the end is empty and enters the combine as O = 0,
  LSE = -inf.  Each split writes its partial O and its own LSE into a
  split-major slot; a combine merges them.
* The FP8 kernel's own amax of O stands down under a split (a max over
  partials over-reports the recombined output): the combine owns the amax of
  the recombined O.  An attention sink, when present, counts exactly once.

Readings taken where the page is silent (each stated again where it is used):
  R1  Q, K and V are e4m3fn codes with one float32 descale factor per tensor:
      value = e4m3(code) * descale.  The output O is bf16 (or float32).
  R2  Scores s_ij = softmax_scale * <q_i, k_j> over the 128 dimensions; O is
      the softmax-weighted sum of the V rows; LSE = ln sum_j exp(s_ij)
      (natural log, the usual log-sum-exp of a softmax's statistics).
  R3  The causal mask is aligned to the bottom-right corner: query row i of a
      batch with sq query rows and skv keys sees keys j <= i + (skv - sq).
      Without the mask every row sees all skv keys.  A row that sees no key
      has O = 0 and LSE = -inf.
  R4  Query tiles are q_tile consecutive rows (the last may be short); KV
      blocks are kv_block consecutive keys.  A tile's KV range is the keys
      its last row may see, [0, min(skv, last + skv - sq + 1)) under the mask,
      in ceil(end / kv_block) blocks; split s of S takes blocks
      [s*base + min(s, rem), ... + base + (s < rem)), base, rem = divmod(n, S).
      Inside a split every row still applies its own mask.
  R5  Query head h reads KV head h // (h_q / h_kv).
  R6  Sink: one extra key per query head with logit sink[h] (natural-log
      units, not scaled) and a zero value row, applied once, in the combine:
      O <- O / (1 + exp(sink[h] - LSE)); the returned LSE excludes it.
  R7  amax = max |O| over every valid output element of the tensor, taken on
      the recombined output with the sink applied, before the cast.

Shapes (numpy arrays, padded "batch, sequence, head, dim" layout):
  q  [B, Sq_max, h_q, 128], k and v [B, Skv_max, h_kv, 128]  (float values)
  seqlen_q [B], seqlen_kv [B]  (rows / keys actually present per batch)
  O  [B, Sq_max, h_q, 128], LSE [B, Sq_max, h_q]; rows past seqlen_q are
  left at O = 0, LSE = -inf (they are not part of the result).
"""

import math

import numpy as np

from .smla_oracle import e4m3_decode, split_block_ranges

D = 128


def dequantize(codes, descale):
    """R1: e4m3fn codes times one float32 descale factor per tensor, in float64."""
    return e4m3_decode(codes) * float(np.float32(descale))


def visible_keys(i, sq, skv, causal):
    """R3: number of leading keys query row i may see (0 .. skv)."""
    if not causal:
        return skv
    return int(min(skv, max(0, i + (skv - sq) + 1)))


def kv_head(h, h_q, h_kv):
    """R5: the KV head that query head h reads (h_q / h_kv query heads per KV head)."""
    return h // (h_q // h_kv)


def attend_rows(qrows, krows, vrows, scale, nvis):
    """Softmax attention of query rows over key rows, row r seeing keys [0, nvis[r]).

    qrows [n, d], krows / vrows [m, d] (d = 128 in the workloads; any d here).
    Returns (O [n, d], LSE [n]); a row that sees no key gets O = 0, LSE = -inf.
    """
    n = qrows.shape[0]
    O = np.zeros((n, vrows.shape[1]))
    L = np.full(n, -np.inf)
    for r in range(n):
        m = int(nvis[r])
        if m <= 0:
            continue
        s = float(scale) * (krows[:m] @ qrows[r])            # [m]
        mx = s.max()
        e = np.exp(s - mx)
        l = e.sum()
        O[r] = (e @ vrows[:m]) / l
        L[r] = mx + math.log(l)
    return O, L


def prefill(q, k, v, seqlen_q, seqlen_kv, scale, causal=True):
    """Final O and LSE (no sink) by the plain definition, R2-R5."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, _, h_q, _ = q.shape
    h_kv = k.shape[2]
    O = np.zeros(q.shape)
    L = np.full(q.shape[:3], -np.inf)
    for b in range(B):
        sq, skv = int(seqlen_q[b]), int(seqlen_kv[b])
        nvis = [visible_keys(i, sq, skv, causal) for i in range(sq)]
        for h in range(h_q):
            hk = kv_head(h, h_q, h_kv)
            O[b, :sq, h], L[b, :sq, h] = attend_rows(q[b, :sq, h], k[b, :skv, hk], v[b, :skv, hk], scale, nvis)
    return O, L


def tile_block_count(tile, sq, skv, causal, q_tile, kv_block):
    """R4: KV blocks in the masked range of query tile `tile` (rows tile*q_tile ..)."""
    last = min(sq, (tile + 1) * q_tile) - 1
    end = visible_keys(last, sq, skv, causal)
    return -(-end // kv_block)


def prefill_split_partials(q, k, v, seqlen_q, seqlen_kv, scale, num_splits, causal=True, q_tile=64, kv_block=64):
    """Split-major partials, R4: o [S, B, Sq_max, h_q, 128], lse [S, B, Sq_max, h_q].

    Split s of row i covers the keys of its tile's split-s block range, and of
    those only the ones row i may see; no such key: (0, -inf).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, _, h_q, _ = q.shape
    h_kv = k.shape[2]
    o_part = np.zeros((num_splits,) + q.shape)
    l_part = np.full((num_splits,) + q.shape[:3], -np.inf)
    for b in range(B):
        sq, skv = int(seqlen_q[b]), int(seqlen_kv[b])
        for tile in range(-(-sq // q_tile)):
            rows = range(tile * q_tile, min(sq, (tile + 1) * q_tile))
            n_blk = tile_block_count(tile, sq, skv, causal, q_tile, kv_block)
            for s, (b0, b1) in enumerate(split_block_ranges(n_blk, num_splits)):
                j0, j1 = min(skv, b0 * kv_block), min(skv, b1 * kv_block)
                for i in rows:
                    m = visible_keys(i, sq, skv, causal)
                    hi = min(j1, m)
                    if hi <= j0:
                        continue
                    for h in range(h_q):
                        hk = kv_head(h, h_q, h_kv)
                        o, l = attend_rows(q[b, i:i + 1, h], k[b, j0:hi, hk], v[b, j0:hi, hk], scale, [hi - j0])
                        o_part[s, b, i, h], l_part[s, b, i, h] = o[0], l[0]
    return o_part, l_part


def combine_ln(o_part, l_part):
    """Merge split partials (natural-log LSEs): M = max_s LSE_s, w_s = exp(LSE_s - M),
    O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s; every split at -inf gives
    O = 0, LSE = -inf."""
    o_part = np.asarray(o_part, np.float64)
    l_part = np.asarray(l_part, np.float64)
    M = l_part.max(axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(l_part), 0.0, np.exp(l_part - Ms[None]))
    ws = w.sum(axis=0)
    wss = np.where(empty, 1.0, ws)
    O = (w[..., None] * o_part).sum(axis=0) / wss[..., None]
    O[empty] = 0.0
    L = np.where(empty, -np.inf, Ms + np.log(wss))
    return O, L


def apply_sink_ln(O, L, sink):
    """R6: O * 1 / (1 + exp(sink[h] - LSE)); rows with LSE = -inf stay 0."""
    if sink is None:
        return np.array(O, np.float64)
    O = np.asarray(O, np.float64)
    L = np.asarray(L, np.float64)
    with np.errstate(over="ignore"):
        f = 1.0 / (1.0 + np.exp(np.asarray(sink, np.float64)[None, None, :] - L))
    f = np.where(np.isneginf(L), 0.0, f)
    return O * f[..., None]


def output_amax(O, seqlen_q):
    """R7: largest |O| over the valid rows of every batch (0 when there are none)."""
    a = 0.0
    for b in range(O.shape[0]):
        sq = int(seqlen_q[b])
        if sq > 0:
            a = max(a, float(np.abs(O[b, :sq]).max()))
    return a
