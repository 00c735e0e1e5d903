"""Pins of the float64 oracle against things other than itself.

Each check ties the oracle to a brute-force evaluation, a closed form, an
invariant, a library routine or a figure the pages print, so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails at
least one of them.  CPU only.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import smla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN2 = math.log(2.0)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _rand_case(seed, s_q=2, h_q=2, n_pool=16, topk=8, d=576):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((s_q, h_q, d)))
    kv = _bf16(rng.standard_normal((n_pool, d)))
    idx = np.stack([rng.choice(n_pool, topk, replace=False) for _ in range(s_q)]).astype(np.int32)
    return q, kv, idx


# ---------------------------------------------------------------------------
# brute force at 50 digits
# ---------------------------------------------------------------------------
def _mp_attention(q, kv, idx, n_pool, scale, sink=None):
    """Full-softmax attention written out in mpmath (50 digits), one token at a time."""
    mpmath.mp.dps = 50
    s_q, h_q = q.shape[0], q.shape[1]
    O_out = np.zeros((s_q, h_q, 512))
    L_out = np.zeros((s_q, h_q))
    for t in range(s_q):
        rows = [int(r) for r in idx[t] if 0 <= int(r) < n_pool]
        for h in range(h_q):
            if not rows:
                O_out[t, h] = 0.0
                L_out[t, h] = -np.inf
                continue
            qv = [mpmath.mpf(float(x)) for x in q[t, h]]
            scores = []
            for r in rows:
                kr = kv[r]
                acc = mpmath.mpf(0)
                for a, b in zip(qv, kr):
                    acc += a * mpmath.mpf(float(b))
                scores.append(mpmath.mpf(float(scale)) * acc)
            ex = [mpmath.e ** s for s in scores]
            denom = mpmath.fsum(ex)
            full = denom + (mpmath.e ** mpmath.mpf(float(sink[h])) if sink is not None else 0)
            for c in range(512):
                num = mpmath.fsum(e * mpmath.mpf(float(kv[r][c])) for e, r in zip(ex, rows))
                O_out[t, h, c] = float(num / full)
            L_out[t, h] = float(mpmath.log(denom) / mpmath.log(2))
    return O_out, L_out


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_mpmath(seed):
    q, kv, idx = _rand_case(seed)
    idx[0, 3] = -1
    idx[1, 0] = 16          # out of range: masked
    idx[1, 5] = -7
    sink = np.array([0.3, -1.2])
    scale = float(np.float32(1 / 24))
    ref_O, ref_L = _mp_attention(q, kv, idx, 16, scale, sink)
    got_O, got_L = O.decode(q, kv, idx, 16, scale, sink)
    assert np.max(np.abs(got_O - ref_O)) <= 1e-12
    assert np.max(np.abs(got_L - ref_L)) <= 1e-12
    for S in (2, 3):
        got_O, got_L = O.decode_split(q, kv, idx, 16, scale, S, split_block=2, sink=sink)
        assert np.max(np.abs(got_O - ref_O)) <= 1e-12
        assert np.max(np.abs(got_L - ref_L)) <= 1e-12


def test_brute_force_partials():
    """Each partial is the normalised attention over its own slot range only."""
    q, kv, idx = _rand_case(5, topk=8)
    idx[0, 6] = -1
    scale = 0.05
    o_acc, lse_acc = O.split_partials(q, kv, idx, 16, scale, num_splits=3, split_block=2)
    # 4 blocks of 2 slots over 3 splits: slots [0,4), [4,6), [6,8)
    for s, (i0, i1) in enumerate([(0, 4), (4, 6), (6, 8)]):
        ref_O, ref_L = _mp_attention(q, kv, idx[:, i0:i1], 16, scale)
        assert np.max(np.abs(o_acc[s] - ref_O)) <= 1e-12
        assert np.max(np.abs(lse_acc[s] - ref_L)) <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_zero_query_gives_mean_of_values():
    q, kv, idx = _rand_case(2, s_q=1, h_q=3, n_pool=32, topk=10)
    q[:] = 0.0
    idx[0, [1, 4]] = -1
    rows = idx[0][idx[0] >= 0]
    got_O, got_L = O.decode(q, kv, idx, 32, 1 / 24)
    np.testing.assert_allclose(got_O[0], np.tile(kv[rows, :512].mean(axis=0), (3, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_L[0], np.full(3, math.log2(len(rows))), rtol=0, atol=1e-13)


def test_equal_scores_from_shared_rope_part():
    """Latent query part zero, every row sharing its RoPE part: all scores equal c."""
    rng = np.random.default_rng(3)
    n_pool, k, h = 40, 12, 4
    kv = _bf16(rng.standard_normal((n_pool, 576)))
    rope = _bf16(rng.standard_normal(64))
    kv[:, 512:] = rope
    q = _bf16(rng.standard_normal((1, h, 576)))
    q[:, :, :512] = 0.0
    idx = rng.choice(n_pool, k, replace=False)[None].astype(np.int32)
    scale = 1 / 24
    c = scale * (q[0, :, 512:].astype(np.float64) @ rope.astype(np.float64))     # [h]
    got_O, got_L = O.decode(q, kv, idx, n_pool, scale)
    mean_v = kv[idx[0], :512].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(got_O[0], np.tile(mean_v, (h, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_L[0], math.log2(k) + c / LN2, rtol=0, atol=1e-12)
    # the sink on equal scores: mean V * k e^c / (k e^c + e^sink)
    sink = np.array([0.5, -2.0, 1.5, 0.0])
    got_O, _ = O.decode(q, kv, idx, n_pool, scale, sink)
    f = k * np.exp(c) / (k * np.exp(c) + np.exp(sink))
    np.testing.assert_allclose(got_O[0], f[:, None] * mean_v[None], rtol=0, atol=1e-13)


def test_identical_rows():
    rng = np.random.default_rng(4)
    row = _bf16(rng.standard_normal(576))
    kv = np.tile(row, (20, 1))
    q = _bf16(rng.standard_normal((2, 3, 576)))
    idx = np.array([[0, 5, 9, -1, 13], [2, 3, 4, 6, 7]], dtype=np.int32)
    scale = 1 / 24
    got_O, got_L = O.decode(q, kv, idx, 20, scale)
    c = scale * (q.astype(np.float64) @ row.astype(np.float64))                # [2, 3]
    np.testing.assert_allclose(got_O, np.broadcast_to(row[:512], got_O.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_L, np.log2([[4], [5]]) + c / LN2, rtol=0, atol=1e-12)


def test_single_valid_slot():
    q, kv, idx = _rand_case(6, s_q=1, h_q=2, n_pool=16, topk=5)
    idx[0, [0, 1, 3, 4]] = -1
    j = int(idx[0, 2])
    scale = 1 / 24
    got_O, got_L = O.decode(q, kv, idx, 16, scale)
    s = scale * (q[0].astype(np.float64) @ kv[j].astype(np.float64))
    np.testing.assert_allclose(got_O[0], np.tile(kv[j, :512], (2, 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(got_L[0], s / LN2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("sink", [None, np.array([0.7, -0.1])])
def test_all_slots_masked(sink):
    q, kv, idx = _rand_case(7, s_q=1, h_q=2, n_pool=16, topk=6)
    idx[:] = -1
    idx[0, 2] = 16
    for got_O, got_L in (O.decode(q, kv, idx, 16, 0.1, sink),
                         O.decode_split(q, kv, idx, 16, 0.1, 3, split_block=2, sink=sink)):
        assert np.all(got_O == 0.0)
        assert np.all(np.isneginf(got_L))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 4, 7, 8, 16])
def test_split_invariance(S):
    q, kv, idx = _rand_case(8, s_q=3, h_q=4, n_pool=300, topk=150)
    idx[1, ::7] = -1
    idx[2, :] = -1                     # a token with nothing valid
    sink = np.array([0.1, -0.4, 2.0, -3.0])
    ref_O, ref_L = O.decode(q, kv, idx, 300, 1 / 24, sink)
    got_O, got_L = O.decode_split(q, kv, idx, 300, 1 / 24, S, split_block=16, sink=sink)
    assert np.max(np.abs(got_O - ref_O)) <= 1e-12
    fin = np.isfinite(ref_L)
    assert np.array_equal(fin, np.isfinite(got_L))
    assert np.max(np.abs(got_L[fin] - ref_L[fin])) <= 1e-12


def test_slot_permutation_and_padding_insertion():
    q, kv, idx = _rand_case(9, s_q=2, h_q=3, n_pool=200, topk=40)
    ref_O, ref_L = O.decode_split(q, kv, idx, 200, 1 / 24, 4, split_block=8)
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(40) for _ in range(2)])
    idx_p = np.take_along_axis(idx, perm, axis=1)
    got_O, got_L = O.decode_split(q, kv, idx_p, 200, 1 / 24, 4, split_block=8)
    assert np.max(np.abs(got_O - ref_O)) <= 1e-12 and np.max(np.abs(got_L - ref_L)) <= 1e-12
    idx_pad = np.full((2, 57), -1, dtype=np.int32)
    pos = np.sort(rng.choice(57, 40, replace=False))
    idx_pad[:, pos] = idx
    got_O, got_L = O.decode_split(q, kv, idx_pad, 200, 1 / 24, 3, split_block=8)
    assert np.max(np.abs(got_O - ref_O)) <= 1e-12 and np.max(np.abs(got_L - ref_L)) <= 1e-12


def test_minus_inf_sink_is_no_sink():
    q, kv, idx = _rand_case(10, s_q=2, h_q=2, n_pool=64, topk=20)
    a, _ = O.decode(q, kv, idx, 64, 1 / 24, np.array([-np.inf, -np.inf]))
    b, _ = O.decode(q, kv, idx, 64, 1 / 24, None)
    assert np.array_equal(a, b)


def test_sink_factor_bounds():
    """A sink only shrinks each output row, by a factor in (0, 1), the same for every column."""
    q, kv, idx = _rand_case(11, s_q=1, h_q=4, n_pool=64, topk=20)
    sink = np.array([-5.0, 0.0, 3.0, 10.0])
    a, _ = O.decode(q, kv, idx, 64, 1 / 24, sink)
    b, _ = O.decode(q, kv, idx, 64, 1 / 24, None)
    ratio = a / b
    assert np.all((ratio > 0) & (ratio < 1))
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-12, atol=0)
    assert np.all(np.diff(ratio[0, :, 0]) < 0)         # larger sink, smaller factor


def test_combine_of_single_split_is_identity():
    rng = np.random.default_rng(12)
    o = rng.standard_normal((1, 3, 4, 512))
    lse = rng.standard_normal((1, 3, 4)) * 5
    got_O, got_L = O.combine_partials(o, lse)
    assert np.max(np.abs(got_O - o[0])) <= 1e-15 and np.max(np.abs(got_L - lse[0])) <= 1e-14


def test_combine_equal_lse_is_plain_mean_and_empty_splits_drop_out():
    rng = np.random.default_rng(13)
    o = rng.standard_normal((4, 2, 3, 512))
    lse = np.full((4, 2, 3), 1.25)
    lse[3] = -np.inf                     # an empty split contributes nothing
    o[3] = 0.0
    got_O, got_L = O.combine_partials(o, lse)
    np.testing.assert_allclose(got_O, o[:3].mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(got_L, 1.25 + math.log2(3), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# library special case: the whole tiny pool selected == dense attention
# ---------------------------------------------------------------------------
def test_dense_special_case_against_torch_sdpa():
    rng = np.random.default_rng(14)
    n_pool, h = 24, 4
    q = _bf16(rng.standard_normal((2, h, 576)))
    kv = _bf16(rng.standard_normal((n_pool, 576)))
    idx = np.stack([rng.permutation(n_pool) for _ in range(2)]).astype(np.int32)
    sink = np.array([0.3, -1.0, 2.5, 0.0])
    scale = float(np.float32(1 / 24))
    got_O, got_L = O.decode(q, kv, idx, n_pool, scale, sink)
    qt = torch.from_numpy(q.astype(np.float64))                       # [2, h, 576]
    K = torch.from_numpy(kv.astype(np.float64))                       # [n, 576]
    V = K[:, :512]
    # dense attention with one extra zero key/value whose additive mask is the sink
    Kx = torch.cat([K, torch.zeros(1, 576, dtype=torch.float64)])
    Vx = torch.cat([V, torch.zeros(1, 512, dtype=torch.float64)])
    mask = torch.zeros(h, n_pool + 1, dtype=torch.float64)
    mask[:, -1] = torch.from_numpy(sink)
    for t in range(2):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[t][None], Kx[None].contiguous(), Vx[None].contiguous(), attn_mask=mask[None], scale=scale)[0]
        assert torch.max(torch.abs(ref - torch.from_numpy(got_O[t]))).item() <= 1e-13
        lse = torch.logsumexp(scale * (qt[t] @ K.T), dim=-1) / LN2
        assert torch.max(torch.abs(lse - torch.from_numpy(got_L[t]))).item() <= 1e-13


# ---------------------------------------------------------------------------
# split partition rule
# ---------------------------------------------------------------------------
def test_partition_worked_examples():
    # 640 slots in 64-slot blocks = 10 blocks
    assert O.split_block_ranges(10, 1) == [(0, 10)]
    assert O.split_block_ranges(10, 2) == [(0, 5), (5, 10)]
    assert O.split_block_ranges(10, 3) == [(0, 4), (4, 7), (7, 10)]
    assert O.split_block_ranges(10, 4) == [(0, 3), (3, 6), (6, 8), (8, 10)]
    assert O.split_block_ranges(10, 16) == [(b, b + 1) for b in range(10)] + [(10, 10)] * 6
    assert O.split_slot_ranges(640, 64, 4) == [(0, 192), (192, 384), (384, 512), (512, 640)]
    assert O.split_slot_ranges(64, 64, 16) == [(0, 64)] + [(64, 64)] * 15
    assert O.split_slot_ranges(100, 64, 2) == [(0, 64), (64, 100)]          # ragged last block


@pytest.mark.parametrize("n_blocks", [0, 1, 5, 10, 17, 64])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 16, 33])
def test_partition_properties(n_blocks, S):
    r = O.split_block_ranges(n_blocks, S)
    assert len(r) == S and r[0][0] == 0 and r[-1][1] == n_blocks
    assert all(r[i][1] == r[i + 1][0] for i in range(S - 1))
    sizes = [b - a for a, b in r]
    assert max(sizes) - min(sizes) <= 1
    assert sizes == sorted(sizes, reverse=True)


def test_partial_bytes_printed_figures():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "partial_bytes.txt")) if l.strip() and not l.startswith("#")]
    assert rows
    for s_q, h_q, d_v, S, mb in rows:
        s_q, h_q, d_v, S = int(s_q), int(h_q), int(d_v), int(S)
        o_bytes = O.partial_bytes(s_q, h_q, S, d_v) - S * s_q * h_q * 4     # drop the LSE part
        digits = len(mb.split(".")[1])
        assert round(o_bytes / 1e6, digits) == float(mb)


# ---------------------------------------------------------------------------
# e4m3
# ---------------------------------------------------------------------------
def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert O.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert O.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6


def test_e4m3_encode_against_torch_in_range():
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (vals[1:] + vals[:-1]) / 2                   # exact ties: round to even
    rng = np.random.default_rng(15)
    rand = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-12, 1, 20000))
    x = np.concatenate([vals, -vals, mids, -mids, mids * (1 + 1e-9), mids * (1 - 1e-9), rand])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates_and_keeps_sign():
    got = O.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, -1e6, -0.0, 0.0, -1e-9]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


def test_fp8_per_token_scale():
    O_ = np.zeros((3, 2, 512))
    O_[0, 1, 7] = -3.5
    O_[1, 0, 0] = 0.25
    codes, scale = O.fp8_quantize_per_token(O_)
    assert scale.tolist() == [3.5 / 448, 0.25 / 448, 1.0]
    assert codes[0, 1, 7] == 0xFE and codes[1, 0, 0] == 0x7E and not codes[2].any()
    c32, s32 = O.fp8_quantize_per_token_f32(O_.astype(np.float32))
    assert np.array_equal(codes, c32) and np.allclose(scale, s32, rtol=1e-7)


def _fp8_tie_heavy_tokens(seed=5, per_token=4096):
    """Float32 tokens whose elements sit on exact e4m3 midpoints once divided by the
    token's float32 scale (amax / 448, not a power of two), so that the rounding
    decision depends on the precision in which O / scale is formed."""
    rng = np.random.default_rng(seed)
    vals = O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    toks = []
    for _ in range(6):
        amax = np.float32(448.0 * rng.uniform(0.3, 3.0))
        s = np.float32(amax / np.float32(448.0))
        m = rng.choice(mids, per_token) * rng.choice([-1.0, 1.0], per_token)
        x = (m * np.float64(s)).astype(np.float32)
        x = np.where(np.abs(x) < amax, x, np.float32(0.0))
        x[0] = amax                                     # the token's amax is exactly amax
        toks.append(x)
    return np.stack(toks).reshape(6, -1, 512)


def _torch_fp8_quantize_f32(O32):
    """Per-token FP8 quantisation in torch float32: amax, amax / 448, O / scale, and
    torch's own e4m3fn cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(O32, dtype=np.float32))
    amax = t.abs().reshape(t.shape[0], -1).amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    ratio = (t / scale[:, None, None]).clamp(-448.0, 448.0)
    return ratio.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), scale.numpy()


def test_fp8_quantize_f32_against_torch_float32():
    """The float32-decided quantisation against torch float32 arithmetic (IEEE division)
    and torch's e4m3fn cast, on random tokens of several magnitudes and on tie-heavy
    tokens where float32 and float64 decide differently."""
    rng = np.random.default_rng(17)
    rand = (rng.standard_normal((5, 64, 512)) * np.array([1e-3, 0.05, 1.0, 7.0, 300.0])[:, None, None])
    rand = rand.astype(np.float32)
    rand[2, 3, ::5] = -0.0
    ties = _fp8_tie_heavy_tokens()
    zero = np.zeros((1, 2, 512), dtype=np.float32)
    for O32 in (rand, ties, zero):
        codes, scale = O.fp8_quantize_per_token_f32(O32)
        ref_codes, ref_scale = _torch_fp8_quantize_f32(O32)
        assert scale.dtype == np.float32 and np.array_equal(scale, ref_scale)
        assert np.array_equal(codes, ref_codes)
    # the tie-heavy tokens do separate the two precisions (the pin is sensitive to them)
    c64, _ = O.fp8_quantize_per_token(ties.astype(np.float64))
    assert int((c64 != _torch_fp8_quantize_f32(ties)[0]).sum()) > 1000


def test_fp8_pool_dequantisation():
    codes = np.array([[0x38, 0xB8, 0x00, 0x7E]], dtype=np.uint8)      # 1, -1, 0, 448
    got = O.dequantize_fp8_rows(codes, np.array([0.5]))
    assert got.tolist() == [[0.5, -0.5, 0.0, 224.0]]
    pool = O.Fp8Pool(np.tile(codes, (3, 1)), np.array([1.0, 2.0, 4.0]))
    assert pool[np.array([2, 0])].tolist() == [[4.0, -4.0, 0.0, 1792.0], [1.0, -1.0, 0.0, 448.0]]
