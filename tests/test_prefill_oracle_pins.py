"""Pins of the float64 prefill oracle (oracle/prefill_oracle.py) against things
other than itself: brute force at 50 digits, closed forms, torch's float64
scaled_dot_product_attention with explicit masks and repeated KV heads, split
invariance, the sink counted once, the partition rule, and planted mistakes that
some pin must reject.  CPU only."""
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import prefill_oracle as P
from oracle import smla_oracle as O


def _case(seed, B=2, h_q=4, h_kv=2, sq=(5, 3), skv=(7, 4), sq_max=None, skv_max=None, d=128, scale=None):
    rng = np.random.default_rng(seed)
    sq_max = sq_max or max(sq)
    skv_max = skv_max or max(skv)
    q = rng.standard_normal((B, sq_max, h_q, d))
    k = rng.standard_normal((B, skv_max, h_kv, d))
    v = rng.standard_normal((B, skv_max, h_kv, d))
    return q, k, v, np.array(sq), np.array(skv), (scale if scale is not None else 1 / math.sqrt(d))


# ---------------------------------------------------------------------------
# brute force at 50 digits
# ---------------------------------------------------------------------------
def _mp_prefill(q, k, v, sq, skv, scale, causal, sink=None):
    mpmath.mp.dps = 50
    B, _, h_q, d = q.shape
    h_kv = k.shape[2]
    O_ = np.zeros(q.shape)
    L_ = np.full(q.shape[:3], -np.inf)
    for b in range(B):
        for i in range(sq[b]):
            # keys the row may see, written from the mask's definition
            keys = [j for j in range(skv[b]) if (not causal) or j - i <= skv[b] - sq[b]]
            for h in range(h_q):
                hk = h * h_kv // h_q
                if not keys:
                    continue
                sc = [mpmath.mpf(float(scale)) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(c))
                                                            for a, c in zip(q[b, i, h], k[b, j, hk])) for j in keys]
                ex = [mpmath.e ** s for s in sc]
                den = mpmath.fsum(ex)
                lse = mpmath.log(den)
                if sink is not None:
                    den = den + mpmath.e ** mpmath.mpf(float(sink[h]))
                for dd in range(d):
                    O_[b, i, h, dd] = float(mpmath.fsum(e * mpmath.mpf(float(v[b, j, hk, dd]))
                                                        for e, j in zip(ex, keys)) / den)
                L_[b, i, h] = float(lse)
    return O_, L_


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_mpmath(causal):
    q, k, v, sq, skv, scale = _case(1, d=16)
    O_ref, L_ref = _mp_prefill(q, k, v, sq, skv, scale, causal)
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, causal)
    assert np.array_equal(np.isneginf(L_), np.isneginf(L_ref))
    fin = np.isfinite(L_ref)
    assert np.max(np.abs(O_ - O_ref)) <= 1e-12
    assert np.max(np.abs(L_[fin] - L_ref[fin])) <= 1e-12


def test_brute_force_with_sink_through_the_split_path():
    q, k, v, sq, skv, scale = _case(2, d=16)
    sink = np.array([0.3, -1.2, 2.0, 0.0])
    O_ref, L_ref = _mp_prefill(q, k, v, sq, skv, scale, True, sink=sink)
    o, l = P.prefill_split_partials(q, k, v, sq, skv, scale, 3, True, q_tile=2, kv_block=2)
    O_, L_ = P.combine_ln(o, l)
    O_ = P.apply_sink_ln(O_, L_, sink)
    fin = np.isfinite(L_ref)
    assert np.max(np.abs(O_ - O_ref)) <= 1e-12
    assert np.max(np.abs(L_[fin] - L_ref[fin])) <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_zero_query_gives_mean_of_visible_values():
    q, k, v, sq, skv, scale = _case(3, B=1, sq=(6,), skv=(9,))
    q[:] = 0.0
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, True)
    for i in range(6):
        n = i + 3 + 1                              # bottom-right: row i sees keys 0 .. i + 3
        for h in range(4):
            assert np.allclose(O_[0, i, h], v[0, :n, h // 2].mean(axis=0), atol=1e-13)
            assert abs(L_[0, i, h] - math.log(n)) <= 1e-13


def test_first_row_of_a_square_causal_batch_sees_one_key():
    q, k, v, sq, skv, scale = _case(4, B=1, sq=(4,), skv=(4,))
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, True)
    for h in range(4):
        assert np.allclose(O_[0, 0, h], v[0, 0, h // 2], atol=1e-14)
        assert abs(L_[0, 0, h] - scale * float(q[0, 0, h] @ k[0, 0, h // 2])) <= 1e-13


def test_rows_that_see_no_key_are_zero_and_minus_inf():
    # more query rows than keys: under the bottom-right mask the first rows see nothing
    q, k, v, sq, skv, scale = _case(5, B=1, sq=(6,), skv=(3,))
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, True)
    assert np.all(O_[0, :3] == 0.0) and np.all(np.isneginf(L_[0, :3]))
    assert np.all(np.isfinite(L_[0, 3:6]))
    o, l = P.prefill_split_partials(q, k, v, sq, skv, scale, 4, True, q_tile=2, kv_block=1)
    O2, L2 = P.combine_ln(o, l)
    assert np.all(O2[0, :3] == 0.0) and np.all(np.isneginf(L2[0, :3]))


# ---------------------------------------------------------------------------
# library special case: torch float64 SDPA with an explicit mask and repeated KV heads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_sdpa(causal):
    q, k, v, sq, skv, scale = _case(6, B=2, h_q=8, h_kv=2, sq=(37, 20), skv=(50, 20))
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, causal)
    for b in range(2):
        n, m = sq[b], skv[b]
        qt = torch.from_numpy(q[b, :n]).permute(1, 0, 2)                   # [h, n, d]
        kt = torch.from_numpy(k[b, :m]).permute(1, 0, 2).repeat_interleave(4, dim=0)
        vt = torch.from_numpy(v[b, :m]).permute(1, 0, 2).repeat_interleave(4, dim=0)
        if causal:
            mask = torch.ones(n, m, dtype=torch.bool).tril(diagonal=m - n)  # bottom-right aligned
        else:
            mask = torch.ones(n, m, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        logits = (qt @ kt.transpose(1, 2)) * scale
        lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
        assert np.max(np.abs(O_[b, :n].transpose(1, 0, 2) - ref.numpy())) <= 1e-12
        assert np.max(np.abs(L_[b, :n].T - lse.numpy())) <= 1e-12


def test_sink_is_one_extra_key_with_a_zero_value():
    """torch SDPA with one extra zero key / zero value column whose additive mask is the
    sink: the oracle's combine-side sink gives the same output."""
    q, k, v, sq, skv, scale = _case(7, B=1, h_q=4, h_kv=4, sq=(9,), skv=(12,))
    sink = np.array([0.5, -2.0, 1.5, 3.0])
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, True)
    O_s = P.apply_sink_ln(O_, L_, sink)
    n, m = 9, 12
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)
    kt = torch.cat([torch.from_numpy(k[0]).permute(1, 0, 2), torch.zeros(4, 1, 128, dtype=torch.float64)], 1)
    vt = torch.cat([torch.from_numpy(v[0]).permute(1, 0, 2), torch.zeros(4, 1, 128, dtype=torch.float64)], 1)
    bias = torch.zeros(4, n, m + 1, dtype=torch.float64)
    bias[:, :, :m] = torch.where(torch.ones(n, m, dtype=torch.bool).tril(diagonal=m - n), 0.0, -math.inf)
    bias[:, :, m] = torch.from_numpy(sink)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias, scale=scale)
    assert np.max(np.abs(O_s[0].transpose(1, 0, 2) - ref.numpy())) <= 1e-12


# ---------------------------------------------------------------------------
# split invariance, partition, sink once, amax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_split_invariance(S, causal):
    q, k, v, sq, skv, scale = _case(8, B=2, h_q=4, h_kv=1, sq=(13, 7), skv=(29, 7), d=32)
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, causal)
    o, l = P.prefill_split_partials(q, k, v, sq, skv, scale, S, causal, q_tile=4, kv_block=4)
    O2, L2 = P.combine_ln(o, l)
    fin = np.isfinite(L_)
    assert np.array_equal(np.isneginf(L2), np.isneginf(L_))
    assert np.max(np.abs(O2 - O_)) <= 1e-12 and np.max(np.abs(L2[fin] - L_[fin])) <= 1e-12


def test_partials_cover_the_tile_ranges():
    """Per tile, the splits' key ranges are consecutive near-equal block chunks of the
    tile's masked range (remainder first); a split's partial is the attention over its
    own keys, and splits past the range are (0, -inf)."""
    q, k, v, sq, skv, scale = _case(9, B=1, h_q=2, h_kv=2, sq=(8,), skv=(11,), d=16)
    S, qt, kb = 4, 4, 2
    o, l = P.prefill_split_partials(q, k, v, sq, skv, scale, S, True, q_tile=qt, kv_block=kb)
    # tile 0 = rows 0..3: last row 3 sees keys 0..6 -> 7 keys -> 4 blocks of 2 -> one block per split
    assert P.tile_block_count(0, 8, 11, True, qt, kb) == 4
    # tile 1 = rows 4..7: last row sees all 11 keys -> 6 blocks -> splits get 2, 2, 1, 1
    assert P.tile_block_count(1, 8, 11, True, qt, kb) == 6
    assert O.split_block_ranges(6, 4) == [(0, 2), (2, 4), (4, 5), (5, 6)]
    # row 5 (tile 1) sees keys 0..8: split 2 = keys 8..9 -> only key 8 visible
    for h in range(2):
        assert np.allclose(o[2, 0, 5, h], v[0, 8, h], atol=1e-14)
        assert abs(l[2, 0, 5, h] - scale * float(q[0, 5, h] @ k[0, 8, h])) <= 1e-13
        # split 3 = key 10: not visible to row 5 -> empty
        assert np.all(o[3, 0, 5, h] == 0.0) and np.isneginf(l[3, 0, 5, h])
    # more splits than blocks: the trailing ones are empty everywhere
    o8, l8 = P.prefill_split_partials(q, k, v, sq, skv, scale, 8, True, q_tile=qt, kv_block=kb)
    assert np.all(np.isneginf(l8[4:, :, :4])) and np.all(o8[4:, :, :4] == 0.0)


def test_sink_counts_once():
    """The sink folded into every split's partial (a per-split sink) changes the result:
    the oracle's combine-side sink is the only one that matches the plain definition."""
    q, k, v, sq, skv, scale = _case(10, B=1, h_q=2, h_kv=2, sq=(6,), skv=(10,), d=16)
    sink = np.array([1.0, -0.5])
    O_, L_ = P.prefill(q, k, v, sq, skv, scale, True)
    ref = P.apply_sink_ln(O_, L_, sink)
    o, l = P.prefill_split_partials(q, k, v, sq, skv, scale, 3, True, q_tile=2, kv_block=2)
    once = P.apply_sink_ln(*P.combine_ln(o, l), sink)
    assert np.max(np.abs(once - ref)) <= 1e-12
    o_each = np.stack([P.apply_sink_ln(o[s], l[s], sink) for s in range(3)])
    each, _ = P.combine_ln(o_each, l)
    assert np.max(np.abs(each - ref)) > 1e-3


def test_amax_ignores_padding_rows():
    O_ = np.zeros((2, 5, 2, 128))
    O_[0, 1, 1, 7] = -3.0
    O_[1, 0, 0, 0] = 2.0
    O_[1, 4, 0, 0] = 100.0                     # row 4 of batch 1 is padding
    assert P.output_amax(O_, np.array([5, 2])) == 3.0
    assert P.output_amax(O_, np.array([0, 0])) == 0.0


def test_dequantize_is_code_value_times_descale():
    codes = np.array([0x38, 0xB8, 0x00, 0x7E], dtype=np.uint8)      # 1, -1, 0, 448
    assert P.dequantize(codes, 0.25).tolist() == [0.25, -0.25, 0.0, 112.0]
    f32 = float(np.float32(0.1))                                     # the descale is a float32
    assert P.dequantize(codes[:1], 0.1)[0] == f32


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def _visible_top_left(i, sq, skv, causal):
    return skv if not causal else int(min(skv, i + 1))


def _kv_head_modulo(h, h_q, h_kv):
    return h % h_kv


def _tile_first_row(tile, sq, skv, causal, q_tile, kv_block):
    end = P.visible_keys(tile * q_tile, sq, skv, causal)
    return -(-end // kv_block)


def _combine_exp2(o_part, l_part):
    M = l_part.max(axis=0)
    Ms = np.where(np.isneginf(M), 0.0, M)
    w = np.where(np.isneginf(l_part), 0.0, np.exp2(l_part - Ms[None]))
    ws = np.where(w.sum(axis=0) == 0, 1.0, w.sum(axis=0))
    return (w[..., None] * o_part).sum(axis=0) / ws[..., None], Ms + np.log(ws)


def _sink_unflipped(O_, L_, sink):
    if sink is None:
        return np.array(O_, np.float64)
    f = 1.0 / (1.0 + np.exp(L_ - np.asarray(sink)[None, None, :]))
    return O_ * np.where(np.isneginf(L_), 0.0, f)[..., None]


def _ranges_remainder_last(n_blocks, num_splits):
    base, rem = divmod(n_blocks, num_splits)
    out, start = [], 0
    for s in range(num_splits):
        n = base + (1 if s >= num_splits - rem else 0)
        out.append((start, start + n))
        start += n
    return out


MUTANTS = {
    "causal_top_left": ("visible_keys", _visible_top_left),
    "kv_head_modulo": ("kv_head", _kv_head_modulo),
    "tile_range_of_first_row": ("tile_block_count", _tile_first_row),
    "combine_exp2": ("combine_ln", _combine_exp2),
    "sink_sign": ("apply_sink_ln", _sink_unflipped),
    "remainder_last": ("split_block_ranges", _ranges_remainder_last),
}

PINS = [
    lambda: test_brute_force_mpmath(True),
    test_brute_force_with_sink_through_the_split_path,
    test_zero_query_gives_mean_of_visible_values,
    lambda: test_against_torch_sdpa(True),
    test_sink_is_one_extra_key_with_a_zero_value,
    lambda: test_split_invariance(3, True),
    test_partials_cover_the_tile_ranges,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(P, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin)
    assert caught, f"no pin rejects the planted mistake {name}"
