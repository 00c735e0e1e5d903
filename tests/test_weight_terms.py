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

The one-term form is correct only for some inputs, so the kernels keep two
terms everywhere.
"""
import numpy as np

import oracle
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
