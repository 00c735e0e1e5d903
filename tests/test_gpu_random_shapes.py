"""GPU parity over seeded random shapes: token counts, head counts, list lengths,
pool sizes, split counts, padding, sink, pool and output formats drawn at
random, so that every kernel the library picks (for 64 heads: the one-part
kernel, the head halves at 2 parts and the head tiles at 4 or 8; for fewer heads
the 4-wave column-part kernel at 1, 2, 4 or 8 parts; each with and without the
look-ahead gather) and both paths meet the oracle bars on shapes no fixed test
names.  A second set draws more jobs than compute units (s_q from 129 to 390):
the one-part kernel whose wave pairs trade weights, and the last round of at
most half the compute units in more parts (in the same launch for a bf16 pool
and 64 heads, else in a second one).
"""
import numpy as np
import pytest

import oracle
from sparse_mla_decode_top_amd import workloads as W
from tests import _harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 40
N_LARGE = 12


def _case(i):
    rng = np.random.default_rng(1000 + i)
    s_q = int(rng.choice([1, 2, 3, 5, 8, 13, 24, 40, 70]))
    h_q = int(rng.choice([16, 32, 64, 64, 64]))
    topk = int(rng.choice([1, 7, 63, 64, 65, 128, 200, 640, 777, 1024]))
    n_pool = int(max(topk, rng.choice([topk, 1024, 5000, 20000])))
    kv_dtype = "fp8" if rng.random() < 0.25 else "bf16"
    pad = rng.choice([None, "random", "trailing"])
    sink = bool(rng.random() < 0.7)
    n_blk = -(-topk // 64)
    S = int(rng.choice([1, 1, 2, 3, 4, 8, 10, 16, n_blk, n_blk + 3]))
    S = max(1, min(S, 64))
    path = "direct" if S == 1 and rng.random() < 0.5 else "split"
    out = str(rng.choice(["f32", "bf16", "fp8"]))
    return dict(s_q=s_q, h_q=h_q, topk=topk, n_pool=n_pool, kv_dtype=kv_dtype, pad=pad, sink=sink, S=S,
                path=path, out=out, seed=2000 + i)


def _case_large(i):
    rng = np.random.default_rng(5000 + i)
    s_q = int(rng.choice([129, 160, 200, 257, 300, 390]))
    h_q = int(rng.choice([32, 64, 64, 64]))
    topk = int(rng.choice([64, 100, 128, 200, 333]))
    n_pool = int(rng.choice([4096, 20000, 70000]))
    kv_dtype = "fp8" if rng.random() < 0.25 else "bf16"
    pad = rng.choice([None, "random", "trailing"])
    sink = bool(rng.random() < 0.7)
    S = int(rng.choice([1, 1, 2, 3]))
    path = "direct" if S == 1 and rng.random() < 0.6 else "split"
    out = str(rng.choice(["f32", "bf16", "fp8"]))
    return dict(s_q=s_q, h_q=h_q, topk=topk, n_pool=n_pool, kv_dtype=kv_dtype, pad=pad, sink=sink, S=S,
                path=path, out=out, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    _check(i, _case(i))


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_batch_matches_oracle(i):
    _check(i, _case_large(i))


@pytest.mark.parametrize("h_q,s_q,kv_dtype", [(16, 5, "bf16"), (32, 40, "fp8"), (64, 3, "fp8"), (16, 300, "fp8"),
                                               (32, 260, "bf16"), (64, 300, "bf16")])
def test_direct_fp8_output(h_q, s_q, kv_dtype):
    """The direct path with an FP8 output (one workgroup a token, every head and column
    for the token's scale; fewer heads padded), small and larger than the compute units."""
    c = dict(s_q=s_q, h_q=h_q, topk=640, n_pool=20000, kv_dtype=kv_dtype, pad="random", sink=True, S=1,
             path="direct", out="fp8", seed=7000 + s_q + h_q)
    _check(f"fp8-direct-{h_q}-{s_q}", c)


def _check(i, c):
    print(f"[case] {i}: {c}", flush=True)
    inp = W.make_inputs(c["s_q"], c["h_q"], c["n_pool"], c["topk"], c["seed"], kv_dtype=c["kv_dtype"],
                        sink=c["sink"], pad=c["pad"])
    dev = H.DeviceInputs(inp)
    O_ref, L_ref = oracle.attend(inp.q.astype(np.float64), H.oracle_pool(inp), inp.indices, inp.n_pool, inp.scale)
    O_fin = H.oracle_final(inp, O_ref, L_ref)
    res = H.run(dev, c["S"], c["out"], c["path"])
    if c["out"] == "fp8":
        # as the FP8 output test: the token scale within the O bar / 448 of amax / 448,
        # decoded values within half an e4m3 step (of |O| / scale widened by the O bar)
        amax_ref = np.abs(O_fin).reshape(c["s_q"], -1).max(axis=1)
        scale = res["scale"]
        scale_ref = np.where(amax_ref > 0, amax_ref / 448.0, 1.0)
        assert np.all(np.abs(scale - scale_ref) <= H.TOL_O / 448.0 + 1e-7 * scale), "token scale"
        dec = oracle.e4m3_decode(res["codes"]) * scale[:, None, None]
        x_bound = np.abs(O_fin) / scale[:, None, None] + H.TOL_O / scale[:, None, None]
        bound = H.e4m3_half_ulp(x_bound) * scale[:, None, None] + H.TOL_O
        assert not np.any(np.isnan(dec))
        assert np.all(np.abs(dec - O_fin) <= bound), "fp8 value error beyond bound"
    else:
        H.assert_o_close(res["O"], O_fin, rel=2.0 ** -8 if c["out"] == "bf16" else 0.0)
        H.assert_lse_close(res["lse"], L_ref)
