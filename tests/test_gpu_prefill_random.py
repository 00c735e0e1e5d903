"""Seeded random shapes of the split-KV FP8 prefill against the float64 oracle.

Each case draws the batch, the KV heads and the query heads per KV head (one or
two heads a workgroup), padded and present query / key counts (ragged, keys
often not a multiple of 64, sometimes fewer keys than rows), the mask, the split
count (1 .. 12, the direct path when 1), the sink and the output dtype, from
numpy default_rng(3000 + i).  Bars as in test_gpu_prefill: O max-abs <= 2e-3
(bf16 output adds 2^-8 |O|), LSE <= 1e-5, amax within 2e-3.
"""
import numpy as np
import pytest

from sparse_mla_decode_top_amd import workloads as W
from tests import _harness as H
from tests.test_gpu_prefill import Dev, check_final, oracle_of, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    rng = np.random.default_rng(3000 + i)
    B = int(rng.integers(1, 4))
    h_kv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4]))
    sq_max = int(rng.integers(1, 200))
    skv_max = int(rng.integers(1, 700))
    sq = [int(rng.integers(0, sq_max + 1)) if rng.random() < 0.3 else sq_max for _ in range(B)]
    skv = [int(rng.integers(0, skv_max + 1)) if rng.random() < 0.3 else skv_max for _ in range(B)]
    return dict(B=B, h_q=h_kv * group, h_kv=h_kv, sq_max=sq_max, skv_max=skv_max, sq=sq, skv=skv,
                causal=bool(rng.random() < 0.7), S=int(rng.choice([1, 1, 2, 3, 4, 7, 12])),
                sink=bool(rng.random() < 0.6), out=str(rng.choice(["f32", "bf16"])), seed=3000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill_matches_oracle(i):
    c = _case(i)
    print(f"[case] prefill random {i}: {c}", flush=True)
    inp = W.make_prefill_inputs(c["B"], c["h_q"], c["h_kv"], c["sq_max"], c["skv_max"], c["seed"], c["sq"],
                                c["skv"], causal=c["causal"], sink=c["sink"])
    dev = Dev(inp)
    O_ref, L_ref = oracle_of(inp)
    path = "direct" if c["S"] == 1 else "split"
    res = run(dev, c["S"], c["out"], path)
    check_final(inp, res, O_ref, L_ref, rel=2.0 ** -8 if c["out"] == "bf16" else 0.0)
