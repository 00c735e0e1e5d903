"""Shared helpers of the GPU parity tests: upload seeded inputs, call the
library through its binding, and evaluate the float64 oracle on the same
inputs (the oracle only ever sees generator output, never GPU results)."""
import functools

import numpy as np

import oracle
from sparse_mla_decode_top_amd import workloads as W

TOL_O = 2e-3          # max-abs on O for bf16 inputs
TOL_LSE = 1e-5        # max-abs on the log2 LSE
TOL_SPLIT = 1e-5      # combined fp32 O between split counts


class Bf16PoolView:
    """Row-indexable float32 view of a bf16 pool that converts only the rows asked for."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, rows):
        return W.bf16_bits_to_f32(self.bits[rows])


def oracle_pool(inp):
    if inp.kv_dtype == "bf16":
        return Bf16PoolView(inp.kv_bits)
    return oracle.Fp8Pool(inp.kv_codes, inp.kv_scale)


@functools.lru_cache(maxsize=4)
def inputs_for(name, seed):
    return W.make_workload_inputs(W.WORKLOADS[name], seed)


@functools.lru_cache(maxsize=8)
def oracle_direct(name, seed):
    """(O without sink, LSE) of every token by the plain definition."""
    inp = inputs_for(name, seed)
    return oracle.attend(inp.q.astype(np.float64), oracle_pool(inp), inp.indices, inp.n_pool, inp.scale)


def oracle_final(inp, O, lse):
    return oracle.apply_sink(O, lse, None if inp.sink is None else inp.sink.astype(np.float64))


class DeviceInputs:
    def __init__(self, inp, device="cuda"):
        import torch
        self.inp = inp
        self.q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(device)
        if inp.kv_dtype == "bf16":
            self.kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(device)
            self.kv_scale = None
        else:
            self.kv = torch.from_numpy(inp.kv_codes).to(device)
            self.kv_scale = torch.from_numpy(inp.kv_scale).to(device)
        self.indices = torch.from_numpy(inp.indices).to(device)
        self.sink = None if inp.sink is None else torch.from_numpy(inp.sink).to(device)


def run(dev, num_splits, out_dtype="f32", path="split", use_sink=True, want_lse=True, indices=None,
        kv=None):
    """One decode through the C ABI.  path: "split" (partials + combine), "direct"
    (S = 1, fused epilogue) or "partial" (partials only).  Buffers start poisoned
    (NaN / 0x7F) so unwritten elements show up."""
    import torch
    import sparse_mla_decode_top_amd as smla
    inp = dev.inp
    s_q, h_q = inp.s_q, inp.h_q
    d = dev.q.device
    o_acc = lse_acc = None
    if path in ("split", "partial"):
        o_acc = torch.full((num_splits, s_q, h_q, 512), float("nan"), device=d)
        lse_acc = torch.full((num_splits, s_q, h_q), float("nan"), device=d)
    out = out_scale = None
    if path != "partial":
        if out_dtype == "f32":
            out = torch.full((s_q, h_q, 512), float("nan"), device=d)
        elif out_dtype == "bf16":
            out = torch.full((s_q, h_q, 512), float("nan"), device=d, dtype=torch.bfloat16)
        else:
            out = torch.full((s_q, h_q, 512), 0x7F, device=d, dtype=torch.uint8)
            out_scale = torch.full((s_q,), float("nan"), device=d)
    lse_out = torch.full((s_q, h_q), float("nan"), device=d) if (want_lse and out is not None) else None
    smla.sparse_mla_decode(dev.q, dev.kv if kv is None else kv, dev.indices if indices is None else indices,
                           num_splits, inp.scale, kv_scale=dev.kv_scale,
                           sink=dev.sink if use_sink else None, o_accum=o_acc, lse_accum=lse_acc, out=out,
                           out_scale=out_scale, lse_out=lse_out)
    torch.cuda.synchronize()
    res = {}
    if out is not None:
        if out_dtype == "fp8":
            res["codes"] = out.cpu().numpy()
            res["scale"] = out_scale.cpu().numpy().astype(np.float64)
        else:
            res["O"] = out.float().cpu().numpy().astype(np.float64)
    if lse_out is not None:
        res["lse"] = lse_out.cpu().numpy().astype(np.float64)
    if o_acc is not None:
        res["o_acc"] = o_acc.cpu().numpy()
        res["lse_acc"] = lse_acc.cpu().numpy()
    return res


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def assert_lse_close(got, ref, tol=TOL_LSE):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.any(np.isnan(got)), "unwritten or NaN LSE"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf pattern differs"
    if fin.any():
        err = max_abs(got[fin], ref[fin])
        assert err <= tol, f"LSE max-abs error {err:.3g} > {tol}"


# Planted rows (a KV row set to 20 x a query head) give that head log2-unit scores
# near 700, and every other head of a token that gathers such a row scores tens of
# units on it, where N(0, 1) inputs keep |LSE| within 9.4 .. 10.4 and |O| below 0.7
# at every named shape (seeds 0-2).  Float32 rounds a score in proportion to the
# sizes of its products (the spacing of float32 near 700 is 6e-5, above the 1e-5 LSE
# bar by itself), and the summation order of O in proportion to the size of the
# summed rows.  So the heads of tokens that gather a planted row are held to the
# bars relative to their size (LSE: |LSE|; O between split counts: the row's largest
# |O|; at least 1 either way); every other token keeps the absolute bars.
def tokens_gathering(indices, rows):
    """Boolean [s_q]: the tokens whose index list names any of `rows`."""
    return np.isin(np.asarray(indices), np.asarray(list(rows))).any(axis=1)


def assert_lse_close_planted(got, ref, planted, tol=TOL_LSE):
    """assert_lse_close, with the heads of the `planted` tokens held to tol * max(1, |ref|).
    Returns how many finite entries took the relative bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.any(np.isnan(got)), "unwritten or NaN LSE"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf pattern differs"
    fin = np.isfinite(ref)
    big = fin & np.asarray(planted)[:, None]
    small = fin & ~big
    if small.any():
        err = max_abs(got[small], ref[small])
        assert err <= tol, f"LSE max-abs error {err:.3g} > {tol} (tokens without a planted row)"
    if big.any():
        rel = float(np.max(np.abs(got[big] - ref[big]) / np.maximum(1.0, np.abs(ref[big]))))
        assert rel <= tol, f"relative LSE error {rel:.3g} > {tol} (tokens gathering a planted row)"
    return int(big.sum())


def assert_split_close_planted(got, base, planted, tol=TOL_SPLIT):
    """Combined fp32 O of two split counts: the rows (heads) of the `planted` tokens are
    held to tol times max(1, the row's largest |O|), every other row to the absolute tol."""
    got = np.asarray(got, np.float64)
    base = np.asarray(base, np.float64)
    rowmax = np.abs(base).max(axis=-1, keepdims=True)
    rel = np.asarray(planted)[:, None, None] & (rowmax > 1.0)
    scale = np.where(rel, rowmax, 1.0)
    err = np.abs(got - base) / scale
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"split-count difference {worst:.3g} > {tol}"
    return int(rel.sum())


def assert_o_close(got, ref, tol=TOL_O, rel=0.0):
    got = np.asarray(got, np.float64)
    assert not np.any(np.isnan(got)), "unwritten or NaN output"
    bound = tol + rel * np.abs(ref)
    err = np.abs(got - ref)
    worst = float(np.max(err - bound)) if err.size else -1.0
    assert worst <= 0, f"O error exceeds bound by {worst:.3g} (max-abs {float(np.max(err)):.3g})"


def assert_fp8_close(codes, scale, O_fin):
    """FP8 output against the oracle: the per-token scale within TOL_O / 448 of amax / 448,
    and each decoded value within half an e4m3 ulp of O / scale (plus TOL_O) of O."""
    import oracle
    s_q = O_fin.shape[0]
    amax_ref = np.abs(O_fin).reshape(s_q, -1).max(axis=1)
    assert np.all(np.abs(scale - amax_ref / 448.0) <= TOL_O / 448.0 + 1e-7 * scale), "fp8 scale"
    dec = oracle.e4m3_decode(codes) * scale[:, None, None]
    x_bound = np.abs(O_fin) / scale[:, None, None] + TOL_O / scale[:, None, None]
    bound = e4m3_half_ulp(x_bound) * scale[:, None, None] + TOL_O
    assert not np.any(np.isnan(dec)), "NaN fp8 code"
    assert np.all(np.abs(dec - O_fin) <= bound), "fp8 value error beyond bound"


def e4m3_half_ulp(x):
    """Half the spacing of e4m3fn values around |x| (saturating range included)."""
    a = np.maximum(np.abs(x), 2.0 ** -6)
    e = np.floor(np.log2(a))
    return np.exp2(e - 4)
