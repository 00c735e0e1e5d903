"""GPU parity of the split-KV FP8 prefill (sdpa_fp8_prefill through the C ABI)
against the float64 prefill oracle on the same seeded inputs.

Bars: O max-abs <= 2e-3 (f32 output; bf16 output adds 2^-8 |O|), LSE (natural
log) max-abs <= 1e-5, the combined f32 O of different split counts within 1e-5
of each other, amax within 2e-3 of the oracle's, and empty splits / rows that see
no key bit-exact (+0.0, -inf).  Padding rows of K and V hold the e4m3 NaN code:
a read of one would turn an output NaN.
"""
import numpy as np
import pytest

from oracle import prefill_oracle as P
from sparse_mla_decode_top_amd import workloads as W
from tests import _harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


class Dev:
    def __init__(self, inp):
        self.inp = inp
        c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        self.q, self.k, self.v = c(inp.q_codes), c(inp.k_codes), c(inp.v_codes)
        self.sq, self.skv = c(inp.seqlen_q), c(inp.seqlen_kv)
        self.sink = None if inp.sink is None else c(inp.sink)


def oracle_of(inp, split=None):
    q = P.dequantize(inp.q_codes, inp.descale_q)
    k = P.dequantize(inp.k_codes, inp.descale_k)
    v = P.dequantize(inp.v_codes, inp.descale_v)
    for b in range(inp.batch):                       # padding (NaN codes) is never part of the result
        q[b, inp.seqlen_q[b]:] = 0.0
        k[b, inp.seqlen_kv[b]:] = 0.0
        v[b, inp.seqlen_kv[b]:] = 0.0
    if split is not None:
        return P.prefill_split_partials(q, k, v, inp.seqlen_q, inp.seqlen_kv, inp.scale, split, inp.causal)
    return P.prefill(q, k, v, inp.seqlen_q, inp.seqlen_kv, inp.scale, inp.causal)


def run(dev, S, out_dtype="f32", path="split", use_sink=True):
    """path: "split" (partials + combine), "direct" (S = 1, no partials) or "partial"."""
    import sparse_mla_decode_top_amd as smla
    inp = dev.inp
    B, sq, hq = inp.batch, inp.sq_max, inp.h_q
    o_part = lse_part = None
    if path in ("split", "partial"):
        o_part = torch.full((S, B, sq, hq, 128), float("nan"), device="cuda")
        lse_part = torch.full((S, B, sq, hq), float("nan"), device="cuda")
    out = lse = amax = None
    if path != "partial":
        dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = torch.full((B, sq, hq, 128), float("nan"), device="cuda", dtype=dt)
        lse = torch.full((B, sq, hq), float("nan"), device="cuda")
        amax = torch.full((1,), float("nan"), device="cuda")
    smla.sdpa_fp8_prefill(dev.q, dev.k, dev.v, dev.sq, dev.skv, S, inp.scale, inp.descale_q, inp.descale_k,
                          inp.descale_v, causal=inp.causal, sink=dev.sink if use_sink else None, o_part=o_part,
                          lse_part=lse_part, out=out, lse_out=lse, amax_out=amax)
    torch.cuda.synchronize()
    res = {}
    if out is not None:
        res["O"] = out.float().cpu().numpy().astype(np.float64)
        res["lse"] = lse.cpu().numpy().astype(np.float64)
        res["amax"] = float(amax.item())
    if o_part is not None:
        res["o_part"] = o_part.cpu().numpy()
        res["lse_part"] = lse_part.cpu().numpy()
    return res


def valid_rows(inp):
    m = np.zeros((inp.batch, inp.sq_max), bool)
    for b in range(inp.batch):
        m[b, :inp.seqlen_q[b]] = True
    return m


def check_final(inp, res, O_ref, L_ref, rel=0.0, sink=True):
    vr = valid_rows(inp)
    O_fin = P.apply_sink_ln(O_ref, L_ref, inp.sink.astype(np.float64) if (sink and inp.sink is not None) else None)
    H.assert_o_close(res["O"][vr], O_fin[vr], rel=rel)
    H.assert_lse_close(res["lse"][vr], L_ref[vr])
    amax_ref = P.output_amax(O_fin, inp.seqlen_q)
    assert abs(res["amax"] - amax_ref) <= H.TOL_O, (res["amax"], amax_ref)
    return O_fin


CASES = {
    # name: (batch, h_q, h_kv, Sq, Skv, seqlen_q, seqlen_kv, causal)
    "ragged_causal": (2, 8, 2, 130, 300, [130, 77], [300, 77], True),
    "ragged_full": (2, 8, 2, 130, 300, [130, 77], [300, 77], False),
    "more_rows_than_keys": (1, 4, 4, 200, 150, [200], [150], True),
    "gqa8_long": (1, 16, 2, 64, 1000, [64], [1000], True),
    # an odd number of query heads per KV head (one head a workgroup), keys not a multiple of 64
    "gqa3_odd": (2, 6, 2, 100, 333, [100, 65], [333, 200], True),
}
_DEV = {}


def dev_for(name, seed=0):
    key = (name, seed)
    if key not in _DEV:
        _DEV.clear()
        B, hq, hk, sq, skv, lq, lk, causal = CASES[name]
        print(f"[case] prefill {name} seed={seed}", flush=True)
        _DEV[key] = Dev(W.make_prefill_inputs(B, hq, hk, sq, skv, seed, lq, lk, causal=causal))
    return _DEV[key]


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_matches_oracle(name):
    dev = dev_for(name)
    inp = dev.inp
    O_ref, L_ref = oracle_of(inp)
    for S, path in ((1, "direct"), (1, "split"), (2, "split"), (3, "split"), (5, "split")):
        print(f"[case] {name} S={S} {path}", flush=True)
        res = run(dev, S, "f32", path)
        check_final(inp, res, O_ref, L_ref)
    res = run(dev, 3, "bf16", "split")
    check_final(inp, res, O_ref, L_ref, rel=2.0 ** -8)
    res = run(dev, 1, "bf16", "direct")
    check_final(inp, res, O_ref, L_ref, rel=2.0 ** -8)
    res = run(dev, 2, "f32", "split", use_sink=False)
    check_final(inp, res, O_ref, L_ref, sink=False)


@pytest.mark.parametrize("name", ["ragged_causal", "more_rows_than_keys", "gqa3_odd"])
def test_prefill_partials_match_oracle(name):
    """Every split's partial (O normalised by its own denominator, LSE) against the
    oracle's split partials; empty splits and rows that see none of a split's keys are
    exactly O = +0.0, LSE = -inf."""
    dev = dev_for(name)
    inp = dev.inp
    vr = valid_rows(inp)
    for S in (3, 8):
        res = run(dev, S, "f32", "partial")
        o_ref, l_ref = oracle_of(inp, split=S)
        o, l = res["o_part"][:, vr], res["lse_part"][:, vr]
        o_ref, l_ref = o_ref[:, vr], l_ref[:, vr]
        empty = np.isneginf(l_ref)
        assert np.all(o[empty] == 0.0) and not np.any(np.signbit(o[empty]))
        assert np.all(np.isneginf(l[empty]))
        H.assert_o_close(o[~empty], o_ref[~empty])
        H.assert_lse_close(l, l_ref)


@pytest.mark.parametrize("name", ["ragged_causal", "gqa8_long"])
def test_prefill_split_count_invariance(name):
    dev = dev_for(name)
    vr = valid_rows(dev.inp)
    base = run(dev, 1, "f32", "split")
    direct = run(dev, 1, "f32", "direct")
    assert H.max_abs(direct["O"][vr], base["O"][vr]) <= H.TOL_SPLIT
    for S in (2, 3, 4, 7, 16, 64):
        res = run(dev, S, "f32", "split")
        err = H.max_abs(res["O"][vr], base["O"][vr])
        assert err <= H.TOL_SPLIT, f"S={S}: {err:.3g}"
        H.assert_lse_close(res["lse"][vr], base["lse"][vr], H.TOL_SPLIT)


def test_prefill_rows_that_see_no_key():
    """Under the bottom-right mask the first Sq - Skv rows see no key: O = +0, LSE = -inf,
    in both paths; a batch with no rows and one with no keys."""
    dev = Dev(W.make_prefill_inputs(3, 4, 2, 96, 80, 5, [96, 0, 40], [50, 70, 0], causal=True))
    inp = dev.inp
    O_ref, L_ref = oracle_of(inp)
    for S, path in ((1, "direct"), (4, "split")):
        res = run(dev, S, "f32", path)
        check_final(inp, res, O_ref, L_ref)
        assert np.all(res["O"][0, :46] == 0.0) and not np.any(np.signbit(res["O"][0, :46]))
        assert np.all(np.isneginf(res["lse"][0, :46]))
        assert np.all(np.isnan(res["O"][1]))                      # no rows: nothing written
        assert np.all(res["O"][2, :40] == 0.0) and np.all(np.isneginf(res["lse"][2, :40]))


@pytest.mark.parametrize("name", sorted(W.PREFILL_WORKLOADS))
def test_prefill_workload_sampled_rows(name):
    """The measured workloads at full size, in the launch the bench times (the chosen
    split count): sampled rows of every batch (tile edges and random ones) against the
    oracle row by row."""
    import sparse_mla_decode_top_amd as smla
    B, hq, hk, sq, skv, causal = W.PREFILL_WORKLOADS[name]
    print(f"[case] prefill workload {name}", flush=True)
    dev = Dev(W.make_prefill_inputs(B, hq, hk, sq, skv, 0, causal=causal))
    inp = dev.inp
    S = smla.smla_prefill_choose_splits(B, sq, skv, hq, hk, 256)
    res = run(dev, S, "bf16", "split" if S > 1 else "direct")
    q = P.dequantize(inp.q_codes, inp.descale_q)
    k = P.dequantize(inp.k_codes, inp.descale_k)
    v = P.dequantize(inp.v_codes, inp.descale_v)
    rng = np.random.default_rng(1)
    for b in range(B):
        rows = np.unique(np.concatenate([[0, 63, 64, sq - 1], rng.choice(sq, 12, replace=False)]))
        for h in (0, hq // 2 + 1, hq - 1):
            hkv = P.kv_head(h, hq, hk)
            nvis = [P.visible_keys(int(i), sq, skv, causal) for i in rows]
            O_r, L_r = P.attend_rows(q[b, rows, h], k[b, :, hkv], v[b, :, hkv], inp.scale, nvis)
            O_r = O_r / (1.0 + np.exp(float(inp.sink[h]) - L_r))[:, None]
            H.assert_o_close(res["O"][b, rows, h], O_r, rel=2.0 ** -8)
            H.assert_lse_close(res["lse"][b, rows, h], L_r)


@pytest.mark.parametrize("S,path", [(3, "split"), (1, "direct")])
def test_prefill_graph_capture_replays_match_eager(S, path):
    """sdpa_fp8_prefill captured into a HIP graph (split: attention + combine; direct: the
    amax reset + attention): every replay, with eager work in between, equals the eager
    call bit for bit, the amax included."""
    import sparse_mla_decode_top_amd as smla
    dev = dev_for("gqa8_long")
    inp = dev.inp
    B, sq, hq = inp.batch, inp.sq_max, inp.h_q
    o_part = lse_part = None
    if path == "split":
        o_part = torch.empty((S, B, sq, hq, 128), device="cuda")
        lse_part = torch.empty((S, B, sq, hq), device="cuda")
    out = torch.empty((B, sq, hq, 128), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, sq, hq), device="cuda")
    amax = torch.empty((1,), device="cuda")

    def step():
        smla.sdpa_fp8_prefill(dev.q, dev.k, dev.v, dev.sq, dev.skv, S, inp.scale, inp.descale_q, inp.descale_k,
                              inp.descale_v, causal=inp.causal, sink=dev.sink, o_part=o_part, lse_part=lse_part,
                              out=out, lse_out=lse, amax_out=amax)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), amax.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        lse.zero_()
        amax.fill_(1e30)                 # a stale larger value: the replay must reset it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(amax, ref[2])
