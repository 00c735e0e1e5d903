"""Seeded synthetic inputs for split-KV sparse MLA decode.

This module only draws inputs; it holds none of the method's arithmetic.  Both
the HIP path (tests, bench) and the float64 oracle consume what it returns.

Recipe (one ``numpy.random.default_rng(seed)`` per case, draws in this order:
q, kv, indices, padding, sink):

* q  [s_q, h_q, 576]: standard normal float32, rounded to bf16 (nearest-even).
* kv [n_pool, 576]:   standard normal float32, rounded to bf16; or, for the FP8
  pool, per row scale = amax(row)/448 and codes = e4m3(row/scale) with
  round-to-nearest-even (values clamped to +-448 before the cast).
* indices [s_q, topk]: per token ``rng.choice(n_pool, topk, replace=False)``
  (unique, uniform over the pool), int32.
* padding: "random" masks a per-token count ~ U{0..topk/4} of slots at uniform
  positions with -1; "trailing" masks that many trailing slots; "oob" puts
  out-of-range values (-5, n_pool, n_pool+7, 2^31-1, -2^31) into random slots.
* sink [h_q]: standard normal float32 (when enabled).
* softmax scale: float32(1/sqrt(576)).

These stand in for the decode shapes of the pages' workload (DeepSeek-V4.1
Flash under a random 4096/256 serving benchmark, h_q=64 per GPU, top-k
"128+512" = 640 slots), which is not available here.
"""

from dataclasses import dataclass, field

import numpy as np

D_QK = 576
D_V = 512
SOFTMAX_SCALE = float(np.float32(1.0 / np.sqrt(576.0)))


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 value of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_codes_of(x):
    """e4m3fn codes of float32 values already clamped to +-448 (torch's CPU cast, RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class Inputs:
    s_q: int
    h_q: int
    n_pool: int
    topk: int
    kv_dtype: str                      # "bf16" or "fp8"
    scale: float
    q_bits: np.ndarray                 # uint16 [s_q, h_q, 576]
    indices: np.ndarray                # int32 [s_q, topk]
    sink: np.ndarray = None            # float32 [h_q] or None
    kv_bits: np.ndarray = None         # uint16 [n_pool, 576]   (bf16 pool)
    kv_codes: np.ndarray = None        # uint8  [n_pool, 576]   (fp8 pool)
    kv_scale: np.ndarray = None        # float32 [n_pool]       (fp8 pool)
    meta: dict = field(default_factory=dict)

    @property
    def q(self):
        """Query values as float32 (exact bf16 values)."""
        return bf16_bits_to_f32(self.q_bits)

    @property
    def kv(self):
        """Pool values as float32 (bf16 pool only; exact)."""
        return bf16_bits_to_f32(self.kv_bits)


def make_inputs(s_q, h_q, n_pool, topk, seed, kv_dtype="bf16", sink=True, pad=None):
    """Draw one seeded case; see the module docstring for the recipe."""
    if topk > n_pool:
        raise ValueError("topk unique indices need topk <= n_pool")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((s_q, h_q, D_QK), dtype=np.float32)
    q_bits = f32_to_bf16_bits(q)
    kv_bits = kv_codes = kv_scale = None
    kv = rng.standard_normal((n_pool, D_QK), dtype=np.float32)
    if kv_dtype == "bf16":
        kv_bits = f32_to_bf16_bits(kv)
    elif kv_dtype == "fp8":
        amax = np.abs(kv).max(axis=1)
        kv_scale = (amax / np.float32(448.0)).astype(np.float32)
        y = np.clip(kv / kv_scale[:, None], -448.0, 448.0).astype(np.float32)
        kv_codes = _e4m3_codes_of(y)
    else:
        raise ValueError(kv_dtype)
    del kv
    indices = np.empty((s_q, topk), dtype=np.int32)
    for t in range(s_q):
        indices[t] = rng.choice(n_pool, size=topk, replace=False)
    meta = {"pad": pad}
    if pad in ("random", "trailing"):
        counts = rng.integers(0, topk // 4 + 1, size=s_q)
        for t in range(s_q):
            c = int(counts[t])
            if pad == "random":
                pos = rng.choice(topk, size=c, replace=False)
            else:
                pos = np.arange(topk - c, topk)
            indices[t, pos] = -1
        meta["pad_counts"] = counts
    elif pad == "oob":
        bad = np.array([-5, n_pool, n_pool + 7, 2 ** 31 - 1, -2 ** 31], dtype=np.int64)
        for t in range(s_q):
            pos = rng.choice(topk, size=min(topk, 8), replace=False)
            indices[t, pos] = bad[rng.integers(0, bad.size, size=pos.size)].astype(np.int32)
    elif pad is not None:
        raise ValueError(pad)
    sink_arr = rng.standard_normal(h_q, dtype=np.float32) if sink else None
    return Inputs(s_q=s_q, h_q=h_q, n_pool=n_pool, topk=topk, kv_dtype=kv_dtype,
                  scale=SOFTMAX_SCALE, q_bits=q_bits, indices=indices, sink=sink_arr,
                  kv_bits=kv_bits, kv_codes=kv_codes, kv_scale=kv_scale, meta=meta)


@dataclass(frozen=True)
class Workload:
    name: str
    s_q: int
    h_q: int
    n_pool: int
    topk: int
    kv_dtype: str
    sink: bool
    pad: str
    num_splits: tuple       # split counts exercised; () = adaptive
    out_dtype: str = "bf16"


# The five workload families (tiny, single-token, small batch, large batch, FP8).
WORKLOADS = {
    "tiny": Workload("tiny", 2, 16, 4096, 64, "bf16", False, None, (1, 2, 4)),
    "single": Workload("single", 1, 64, 65536, 640, "bf16", True, None, (1, 2, 4, 8, 16)),
    "single_nosink": Workload("single_nosink", 1, 64, 65536, 640, "bf16", False, None, (1, 2, 4, 8, 16)),
    "small6": Workload("small6", 6, 64, 131072, 640, "bf16", True, "random", (1, 2, 4, 8)),
    "small16": Workload("small16", 16, 64, 131072, 640, "bf16", True, "random", (1, 2, 4, 8)),
    "small16_trailing": Workload("small16_trailing", 16, 64, 131072, 640, "bf16", True, "trailing", (1, 2, 4, 8)),
    "degenerate": Workload("degenerate", 6, 64, 131072, 64, "bf16", True, None, (16,)),
    "large96": Workload("large96", 96, 64, 262144, 640, "bf16", True, None, ()),
    "large384": Workload("large384", 384, 64, 262144, 640, "bf16", True, None, ()),
    "fp8_1": Workload("fp8_1", 1, 64, 131072, 640, "fp8", True, None, (8,), "fp8"),
    "fp8_16": Workload("fp8_16", 16, 64, 131072, 640, "fp8", True, None, (8,), "fp8"),
}


def make_workload_inputs(w, seed):
    return make_inputs(w.s_q, w.h_q, w.n_pool, w.topk, seed, kv_dtype=w.kv_dtype,
                       sink=w.sink, pad=w.pad)


# ---------------------------------------------------------------------------
# Split-KV FP8 prefill inputs
# ---------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    batch: int
    h_q: int
    h_kv: int
    sq_max: int
    skv_max: int
    causal: bool
    scale: float
    q_codes: np.ndarray                # uint8 [B, Sq, h_q, 128]
    k_codes: np.ndarray                # uint8 [B, Skv, h_kv, 128]
    v_codes: np.ndarray
    descale_q: float
    descale_k: float
    descale_v: float
    seqlen_q: np.ndarray               # int32 [B]
    seqlen_kv: np.ndarray              # int32 [B]
    sink: np.ndarray = None            # float32 [h_q] or None


def _quantize_per_tensor(x, valid):
    """Per-tensor e4m3 codes of x: descale = amax / 448 over the valid entries (float32),
    codes = RNE e4m3 of x / descale (clamped to +-448); padding entries get the NaN code."""
    amax = float(np.abs(x[valid]).max()) if valid.any() else 1.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = np.clip(x / descale, -448.0, 448.0).astype(np.float32)
    codes = _e4m3_codes_of(y)
    codes[~valid] = 0x7F
    return codes, float(descale)


def make_prefill_inputs(batch, h_q, h_kv, sq_max, skv_max, seed, seqlen_q=None, seqlen_kv=None,
                        causal=True, sink=True):
    """One seeded prefill case.  numpy default_rng(seed), draws in the order q, k, v,
    sink: standard normal float32, quantised per tensor to e4m3 (descale = amax / 448
    over the rows present).  seqlen_q / seqlen_kv default to the padded sizes.  Rows
    past a batch's length (padding) hold the e4m3 NaN code 0x7F, so a read of one
    shows up in the output.  softmax scale = float32(1 / sqrt(128))."""
    rng = np.random.default_rng(seed)
    sq = np.full(batch, sq_max, np.int32) if seqlen_q is None else np.asarray(seqlen_q, np.int32)
    skv = np.full(batch, skv_max, np.int32) if seqlen_kv is None else np.asarray(seqlen_kv, np.int32)
    qv = rng.standard_normal((batch, sq_max, h_q, 128), dtype=np.float32)
    kv = rng.standard_normal((batch, skv_max, h_kv, 128), dtype=np.float32)
    vv = rng.standard_normal((batch, skv_max, h_kv, 128), dtype=np.float32)
    qmask = np.zeros(qv.shape, bool)
    kmask = np.zeros(kv.shape, bool)
    for b in range(batch):
        qmask[b, :sq[b]] = True
        kmask[b, :skv[b]] = True
    q_codes, dq = _quantize_per_tensor(qv, qmask)
    k_codes, dk = _quantize_per_tensor(kv, kmask)
    v_codes, dv = _quantize_per_tensor(vv, kmask)
    sink_arr = rng.standard_normal(h_q, dtype=np.float32) if sink else None
    return PrefillInputs(batch=batch, h_q=h_q, h_kv=h_kv, sq_max=sq_max, skv_max=skv_max, causal=causal,
                         scale=float(np.float32(1.0 / np.sqrt(128.0))), q_codes=q_codes, k_codes=k_codes,
                         v_codes=v_codes, descale_q=dq, descale_k=dk, descale_v=dv, seqlen_q=sq,
                         seqlen_kv=skv, sink=sink_arr)


# Prefill workloads: (batch, h_q, h_kv, Sq, Skv, causal).  "prefill_chunk" is a chunk of
# 256 new tokens per sequence over an 8,192-token cache (the case a split-KV prefill
# serves: few query tiles, long KV ranges); "prefill_full" a whole 4,096-token prompt.
PREFILL_WORKLOADS = {
    "prefill_chunk": (2, 32, 8, 256, 8192, True),
    "prefill_full": (1, 32, 8, 4096, 4096, True),
}
