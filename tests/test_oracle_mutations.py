"""Planted mistakes in the oracle must each fail at least one pin.

Each mutation replaces one oracle function with a plausibly wrong version
(a dropped term, a wrong sign or unit, a wrong slice or index rule) and runs
the pins; the test passes when some pin rejects the mutant.  CPU only.
"""
import math

import numpy as np
import pytest

from oracle import smla_oracle as O
import tests.test_oracle_pins as P

LN2 = math.log(2.0)
_orig_attend_token = O.attend_token
_orig_e4m3_encode = O.e4m3_encode


def _attend_natural_log(q_t, kv, idx_t, n_pool, scale):
    o, l = _orig_attend_token(q_t, kv, idx_t, n_pool, scale)
    return o, l * LN2                                   # LSE left in natural-log units


def _attend_wrong_value_slice(q_t, kv, idx_t, n_pool, scale):
    q_t = np.asarray(q_t, dtype=np.float64)
    rows = np.asarray(idx_t)[O.valid_mask(idx_t, n_pool)]
    if rows.size == 0:
        return np.zeros((q_t.shape[0], O.D_V)), np.full(q_t.shape[0], -np.inf)
    K = np.asarray(kv[rows], dtype=np.float64)
    s = scale * (q_t @ K.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ K[:, 64:]) / l, (m[:, 0] + np.log(l[:, 0])) / LN2     # value taken from the wrong dims


def _attend_no_scale(q_t, kv, idx_t, n_pool, scale):
    return _orig_attend_token(q_t, kv, idx_t, n_pool, 1.0)


def _attend_unnormalised(q_t, kv, idx_t, n_pool, scale):
    o, l = _orig_attend_token(q_t, kv, idx_t, n_pool, scale)
    return o * np.exp2(l)[:, None], l                    # partial not divided by its own l


def _sink_sign_flipped(O_, lse, sink):
    if sink is None:
        return np.array(O_, dtype=np.float64)
    f = 1.0 / (1.0 + np.exp(lse * LN2 - np.asarray(sink)[None, :]))
    return np.asarray(O_) * np.where(np.isneginf(lse), 0.0, f)[..., None]


def _combine_natural_exp(o_acc, lse_acc):
    M = lse_acc.max(axis=0)
    w = np.where(np.isneginf(lse_acc), 0.0, np.exp(lse_acc - np.where(np.isneginf(M), 0, M)[None]))
    ws = np.where(w.sum(axis=0) == 0, 1, w.sum(axis=0))
    return (w[..., None] * o_acc).sum(axis=0) / ws[..., None], M + np.log2(ws)


def _ranges_remainder_last(n_blocks, num_splits):
    base, rem = divmod(n_blocks, num_splits)
    out, start = [], 0
    for s in range(num_splits):
        n = base + (1 if s >= num_splits - rem else 0)
        out.append((start, start + n))
        start += n
    return out


def _valid_off_by_one(indices, n_pool):
    idx = np.asarray(indices)
    return (idx >= 0) & (idx <= n_pool)


def _e4m3_round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    return _orig_e4m3_encode(x + np.sign(x) * np.abs(x) * 2.0 ** -30)


def _fp8_f32_ratio_in_f64(O32):
    O32 = np.asarray(O32, dtype=np.float32)
    amax = np.abs(O32).reshape(O32.shape[0], -1).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    ratio = O32.astype(np.float64) / scale.astype(np.float64)[:, None, None]     # decided in float64
    return O.e4m3_encode(ratio), scale


def _fp8_f32_scale_in_f64(O32):
    O32 = np.asarray(O32, dtype=np.float32)
    amax = np.abs(O32).reshape(O32.shape[0], -1).max(axis=1).astype(np.float64)
    scale = np.where(amax > 0, amax / 448.0, 1.0)                                # never rounded to float32
    ratio = (O32 / scale[:, None, None]).astype(np.float32)
    return O.e4m3_encode(ratio.astype(np.float64)), scale


MUTANTS = {
    "lse_natural_log": ("attend_token", _attend_natural_log),
    "value_wrong_slice": ("attend_token", _attend_wrong_value_slice),
    "scale_dropped": ("attend_token", _attend_no_scale),
    "partial_unnormalised": ("attend_token", _attend_unnormalised),
    "sink_sign_flipped": ("apply_sink", _sink_sign_flipped),
    "combine_natural_exp": ("combine_partials", _combine_natural_exp),
    "partition_remainder_last": ("split_block_ranges", _ranges_remainder_last),
    "valid_off_by_one": ("valid_mask", _valid_off_by_one),
    "e4m3_ties_away": ("e4m3_encode", _e4m3_round_half_up),
    "fp8_f32_ratio_in_f64": ("fp8_quantize_per_token_f32", _fp8_f32_ratio_in_f64),
    "fp8_f32_scale_in_f64": ("fp8_quantize_per_token_f32", _fp8_f32_scale_in_f64),
}

PINS = [
    lambda: P.test_brute_force_mpmath(0),
    P.test_brute_force_partials,
    P.test_zero_query_gives_mean_of_values,
    P.test_equal_scores_from_shared_rope_part,
    P.test_identical_rows,
    P.test_single_valid_slot,
    lambda: P.test_split_invariance(3),
    P.test_partition_worked_examples,
    P.test_dense_special_case_against_torch_sdpa,
    P.test_e4m3_encode_against_torch_in_range,
    P.test_fp8_quantize_f32_against_torch_float32,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError):
            caught.append(pin)
    assert caught, f"no pin rejects the planted mistake {name}"
