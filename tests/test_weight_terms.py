"""Why the PV product takes each softmax weight as two bf16 terms (CPU only).

The attention kernels feed the matrix core bf16 operands, so a float32 weight p
enters PV either as one term bf16(p) or as two, hi = bf16(p) and
lo = bf16(p - hi), which carry p to about 2^-17 relative.  These tests model that
weight arithmetic in numpy: float32 scores in log2 units, the integer frame
p = 2^(t - floor t) * 2^(floor t - M), and PV in float64.  They compare the
result with the float64 oracle on the same inputs.

* On the large-batch workload's random inputs one term stays under the 2e-3
  bar on O, by about a factor of two.
* Two dominant slots whose value rows differ put one term over the bar
  whichever denominator it uses: the float32 weights (what the kernels sum) or
  the rounded ones.  Two terms stay two orders of magnitude inside it.

The one-term form is correct only for some inputs, so the decode kernels keep
two terms everywhere.

The prefill's values are e4m3 codes, which f16 holds exactly, so its PV takes
one f16 weight instead (2^-12 relative, against 2^-9 for one bf16 term).  The
prefill tests below model that: one bf16 term fails the bar on rows that see
few keys, one f16 term passes it; and the weights are taken as 2^(t - M + 14)
so that those down to 2^-28 of a row's largest stay out of f16's subnormals,
whose rounding would depend on the frame and so on the split count.
"""
import numpy as np

import oracle
from oracle import prefill_oracle as PO
from sparse_mla_decode_top_amd import workloads as W

TOL_O = 2e-3


def bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(x, np.float32)))


def pv_model(q, kv, idx, scale, terms, denominator):
    """O [h, 512] of one token whose weights enter PV as `terms` bf16 terms.

    q: [h, 576] float32; kv: [n_pool, 576] float32; idx: [topk] (-1 = masked).
    denominator: "float32" sums the unrounded weights, "rounded" the PV operands.
    """
    rows = kv[idx[idx >= 0]]
    s = (rows.astype(np.float64) @ q.astype(np.float64).T).astype(np.float32)   # [n, h]
    t = (s * np.float32(scale * np.log2(np.e))).astype(np.float32)
    M = np.floor(t.max(axis=0))
    fl = np.floor(t)
    p = (np.exp2(t - fl).astype(np.float32) * np.exp2(fl - M)).astype(np.float32)
    hi = bf16(p)
    w = hi if terms == 1 else hi + bf16(p - hi)
    l = (p if denominator == "float32" else w).astype(np.float64).sum(axis=0)
    return (w.astype(np.float64).T @ rows[:, :512].astype(np.float64)) / l[:, None]


def max_error(inp, tokens, terms, denominator):
    q, kv = inp.q, inp.kv
    O_ref, _ = oracle.attend(q[tokens].astype(np.float64), kv.astype(np.float64), inp.indices[tokens],
                             inp.n_pool, inp.scale)
    return max(float(np.abs(pv_model(q[t], kv, inp.indices[t], inp.scale, terms, denominator) - O_ref[i]).max())
               for i, t in enumerate(tokens))


def dominant_pair_inputs():
    """8 tokens; in each, one head's scores are dominated by two slots (blocks 3 and 6)
    whose key parts score ~12 (a few hundredths apart) and whose value rows are +-3."""
    inp = W.make_inputs(8, 64, 8192, 640, seed=41, sink=False)
    q, kv = inp.q, inp.kv.copy()
    rng = np.random.default_rng(5)
    for t in range(8):
        h = 5 * t
        a, b = int(inp.indices[t, 64 * 3 + 7 * t]), int(inp.indices[t, 64 * 6 + 5 * t])
        v = bf16(rng.choice([-3.0, 3.0], 512))
        for row, beta, val in ((a, 4.5, v), (b, 4.5 + 0.01 * (t + 1), -v)):
            kv[row, :512] = val
            kv[row, 512:] = bf16(beta * q[t, h, 512:])
    inp.kv_bits = W.f32_to_bf16_bits(kv)
    return inp


def test_one_term_passes_on_random_large_batch_inputs():
    inp = W.make_workload_inputs(W.WORKLOADS["large96"], 0)
    tokens = list(range(8))
    e1 = max_error(inp, tokens, 1, "float32")
    e2 = max_error(inp, tokens, 2, "float32")
    assert e1 < TOL_O, e1
    assert e2 < 1e-5, e2


def test_one_term_fails_with_two_dominant_slots():
    inp = dominant_pair_inputs()
    tokens = list(range(8))
    for den in ("float32", "rounded"):
        assert max_error(inp, tokens, 1, den) > TOL_O, den
        assert max_error(inp, tokens, 2, den) < TOL_O / 100, den


# ---- prefill: one f16 weight -------------------------------------------------

def weights(p, form):
    """The PV operand a float32 weight p becomes: one bf16 term, one f16 term, or hi + lo bf16."""
    if form == "bf16":
        return bf16(p).astype(np.float64)
    if form == "f16":
        return p.astype(np.float16).astype(np.float64)
    hi = bf16(p)
    return hi.astype(np.float64) + bf16(p - hi)


def prefill_rows_model(qrows, krows, vrows, scale, nvis, form, shift=14.0, key_range=None):
    """Partial (O normalised by its own l, log2 l + frame) of each row over keys
    [k0, k1) of its visible range, with weights 2^(t - M + shift) in `form`.
    The frame M is the floor of the row's largest scaled score in the range."""
    c = np.float32(scale * np.log2(np.e))
    n = qrows.shape[0]
    O = np.zeros((n, vrows.shape[1]))
    L = np.full(n, -np.inf)
    for r in range(n):
        k0, k1 = (0, int(nvis[r])) if key_range is None else (key_range[0], min(key_range[1], int(nvis[r])))
        if k1 <= k0:
            continue
        s = (krows[k0:k1].astype(np.float64) @ qrows[r].astype(np.float64)).astype(np.float32)
        t = (s * c).astype(np.float32)
        M = np.floor(t.max())
        p = np.exp2(t.astype(np.float64) - M + shift).astype(np.float32)
        l = p.astype(np.float64).sum()
        O[r] = (weights(p, form) @ vrows[k0:k1].astype(np.float64)) / l
        L[r] = M - shift + np.log2(l)
    return O, L


def prefill_case():
    inp = PO_inputs = W.make_prefill_inputs(1, 4, 1, 256, 256, seed=3)
    q = PO.dequantize(inp.q_codes, inp.descale_q)
    k = PO.dequantize(inp.k_codes, inp.descale_k)
    v = PO.dequantize(inp.v_codes, inp.descale_v)
    nvis = [PO.visible_keys(i, 256, 256, True) for i in range(256)]
    return PO_inputs, q[0], k[0, :, 0], v[0, :, 0], nvis


def test_prefill_one_f16_weight_passes_where_one_bf16_weight_fails():
    inp, q, k, v, nvis = prefill_case()
    worst = {"bf16": 0.0, "f16": 0.0, "hilo": 0.0}
    for h in range(4):
        O_ref, _ = PO.attend_rows(q[:, h], k, v, inp.scale, nvis)
        for form in worst:
            O, _ = prefill_rows_model(q[:, h], k, v, inp.scale, nvis, form)
            worst[form] = max(worst[form], float(np.abs(O - O_ref).max()))
    assert worst["bf16"] > TOL_O, worst           # the causal rows that see few keys
    assert worst["f16"] < TOL_O / 2, worst
    assert worst["hilo"] < 2e-5, worst


def merged(parts):
    """Merge (O, log2 l + M) partials by the LSE rule, in float64."""
    Ls = np.stack([L for _, L in parts])
    m = Ls.max(axis=0)
    w = np.exp2(Ls - m)
    return sum(w[i][:, None] * parts[i][0] for i in range(len(parts))) / w.sum(axis=0)[:, None]


def test_prefill_f16_weights_split_invariance_needs_the_shift():
    """One key scores 0.5 (log2 units) and 4,095 score -24.5, all with value rows of ones.
    Unshifted, the small weights 2^-24.5 are f16 subnormals in the whole range and round up
    to 2^-24 together, but in the second split's own frame they are normal, so one and two
    splits disagree well beyond 1e-5; with the 2^14 shift both splits round them alike."""
    n = 4096
    c = 1.0 / np.sqrt(128.0) * np.log2(np.e)
    qrow = np.zeros((1, 128))
    qrow[0, 0] = 1.0
    krows = np.zeros((n, 128))
    krows[:, 0] = -24.5 / c
    krows[5, 0] = 0.5 / c                                        # the dominant key, in the first half
    vrows = np.ones((n, 128))
    scale = 1.0 / np.sqrt(128.0)
    gap = {}
    for shift in (0.0, 14.0):
        one = prefill_rows_model(qrow, krows, vrows, scale, [n], "f16", shift)
        two = merged([prefill_rows_model(qrow, krows, vrows, scale, [n], "f16", shift, (0, n // 2)),
                      prefill_rows_model(qrow, krows, vrows, scale, [n], "f16", shift, (n // 2, n))])
        gap[shift] = float(np.abs(one[0] - two).max())
    assert gap[0.0] > 1e-5, gap
    assert gap[14.0] < 1e-9, gap
