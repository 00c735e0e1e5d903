#!/usr/bin/env python3
"""Benchmark of the split-KV sparse MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the attention kernel
over every (token, split) job plus the combine, on inputs already resident in
HBM.  Steps are replayed from HIP graphs of 64 steps (the pages time their
kernels under CUDA graphs) and cycle through L distinct "layers" --
independent pools, queries and index lists whose pools together exceed the
256 MB last-level cache.  At small s_q the rows that all layers gather (0.74 MB per token and
layer) still fit in that cache and stay there across replays, so the graph
figure is a warm-cache one there; at s_q = 384 the gathered rows exceed it.
cold_us_per_step repeats the step with every cache flushed before it (a 1 GiB
overwrite between steps), so that indices, Q and rows all come from HBM.

Prints ONE JSON line (rank 0, N = 1):
  value        microseconds per step (lower is better) at the single-token
               workload: s_q=1, h_q=64, topk=640, pool 65536 bf16 rows, sink on,
               num_splits from smla_choose_num_splits
  roofline     the attention kernel's algorithmic bytes per launch over its mean
               duration (HIP events on its launch stream), against 8 TB/s
  cold_us_per_step  the same step with the caches flushed before each step
  cpu_baseline the float64 oracle timed on the host cores on the same inputs
  sweep        the same measurement at s_q = 6, 16, 96, 384 and for the FP8
               path, and the split-KV FP8 prefill workloads (context)
"""
import argparse
import hashlib
import json
import os
import sys
import time

_CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_CORES))

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA split-KV decode µs/step + HBM TB/s (h_q=64, topk=640, s_q=1..384)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# Algorithmic bytes per query token (h_q = 64, topk = 640, bf16 pool):
KV_BYTES = 640 * 1152          # gathered rows (576 bf16 each)
Q_BYTES = 64 * 576 * 2
IDX_BYTES = 640 * 4
OUT_BYTES = 64 * 512 * 2       # bf16 output
MAIN_BYTES_PER_TOKEN = KV_BYTES + Q_BYTES + IDX_BYTES     # 813,568: the attention kernel's share
MAIN_BYTES_PER_TOKEN_FP8 = 640 * (576 + 4) + Q_BYTES + IDX_BYTES   # e4m3 rows + row scales: 447,488
STEP_BYTES_PER_TOKEN = MAIN_BYTES_PER_TOKEN + OUT_BYTES   # 879,104
FLOPS_PER_TOKEN = 2 * 64 * 640 * (576 + 512)              # 89,128,960
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_mla_decode_top_amd", "csrc", f)
                  for f in ("smla_kernels.hip", "smla_gfx950.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_kernel_single_token.json")

WORKLOADS = {   # name -> (s_q, n_pool, pool dtype / output dtype, fixed num_splits or 0)
    "single": (1, 65536, "bf16", 0),
    "small6": (6, 131072, "bf16", 0),
    "small16": (16, 131072, "bf16", 0),
    "large96": (96, 262144, "bf16", 0),
    "large384": (384, 262144, "bf16", 0),
    "fp8_1": (1, 131072, "fp8", 8),       # e4m3 pool + row scale, e4m3 output + token scale
    "fp8_16": (16, 131072, "fp8", 8),
}
LLC_BYTES = 256 << 20
LABELS = {"single": "single-token decode", "small6": "small decode batch", "small16": "small decode batch",
          "large96": "large decode batch", "large384": "large decode batch", "fp8_1": "FP8 path",
          "fp8_16": "FP8 path"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="single", choices=sorted(WORKLOADS))
    ap.add_argument("--num-splits", type=int, default=0, help="0 = smla_choose_num_splits")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--prefill-only", action="store_true",
                    help="measure only the split-KV FP8 prefill workloads and print their results as one JSON line")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only a plain 256 MiB device copy (calibrates the HBM byte counters)")
    ap.add_argument("--kernel-stats", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace --stats output directory and exit")
    ap.add_argument("--hbm-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output directories of this bench "
                         "(--no-sweep) and of --copy-only: print the calibrated HBM bytes per launch of the "
                         "attention kernel, write them to the traffic record, and exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc output directories of this bench: print each kernel's counters per "
                         "dispatch (sum and max over the counter's instances) and the MFMA figures, and exit")
    return ap.parse_args()


def source_hash():
    """Hash of the decode kernels' code (their source and the shared device header):
    comments and whitespace removed, so that only a change to the code makes a
    recorded traffic figure stale."""
    import re
    text = ""
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


class Layer:
    """Device-resident inputs of one independent decode layer."""

    def __init__(self, s_q, n_pool, seed, torch, W, dtype="bf16"):
        inp = W.make_inputs(s_q, 64, n_pool, 640, seed, kv_dtype=dtype, sink=True)
        self.inp = inp
        self.q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
        self.indices = torch.from_numpy(inp.indices).cuda()
        self.sink = torch.from_numpy(inp.sink).cuda()
        if dtype == "bf16":
            self.kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).cuda()
            self.kv_scale = None
            self.out = torch.empty((s_q, 64, 512), dtype=torch.bfloat16, device="cuda")
            self.out_scale = None
        else:
            self.kv = torch.from_numpy(inp.kv_codes).cuda()
            self.kv_scale = torch.from_numpy(inp.kv_scale).cuda()
            self.out = torch.empty((s_q, 64, 512), dtype=torch.uint8, device="cuda")
            self.out_scale = torch.empty((s_q,), dtype=torch.float32, device="cuda")


def build_layers(s_q, n_pool, torch, W, seed0=1000, dtype="bf16"):
    per_pool = n_pool * 576 * (2 if dtype == "bf16" else 1)
    n_layers = max(2, -(-2 * LLC_BYTES // per_pool))       # pools total >= 2x the last-level cache
    log(f"s_q={s_q}: generating {n_layers} layers of {per_pool / 1e6:.0f} MB {dtype} pools")
    return [Layer(s_q, n_pool, seed0 + i, torch, W, dtype) for i in range(n_layers)]


GRAPH_STEPS = 64   # steps captured per graph: about the attention calls of one forward of a ~60-layer model


def time_steps(layers, S, steps, warmup, torch, smla):
    """Step time from graph replays, exactly `warmup` untimed then `steps` timed steps.

    Step i of a run calls layer i mod L.  The steps are captured in graphs of GRAPH_STEPS
    steps (rounded up to whole cycles over the layers), plus one graph that holds the
    remainder of each run.  Launching a graph costs about 5 us of GPU time on this
    machine whatever its size; a model's decode graph spreads that over its ~60 layers,
    and so do graphs of this size (one cycle of 8 layers per graph would add about
    0.7 us to every step).  Returns (wall us/step, event us/step, steps, warmup)."""
    s_q = layers[0].inp.s_q
    scale = layers[0].inp.scale
    o_acc = torch.empty((S, s_q, 64, 512), device="cuda") if S > 1 else None
    lse_acc = torch.empty((S, s_q, 64), device="cuda") if S > 1 else None

    def step(L):
        smla.sparse_mla_decode(L.q, L.kv, L.indices, S, scale, kv_scale=L.kv_scale, sink=L.sink, o_accum=o_acc,
                               lse_accum=lse_acc, out=L.out, out_scale=L.out_scale)

    for L in layers:                  # eager warm-up (also loads the library)
        step(L)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L in layers:
            step(L)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    n = len(layers)
    per = n * max(1, -(-GRAPH_STEPS // n))

    def capture(k):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(k):
                step(layers[i % n])
        return g

    g_full = capture(per)
    g_rem = {r: capture(r) for r in {warmup % per, steps % per} if r}

    def replay(k):
        full, rem = divmod(k, per)
        for _ in range(full):
            g_full.replay()
        if rem:
            g_rem[rem].replay()

    replay(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    replay(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e6 / steps, e0.elapsed_time(e1) * 1e3 / steps, steps, warmup


def time_cold(layers, S, steps, torch, smla, flush_bytes=1 << 30):
    """Median step time with the caches flushed before every step: a 1 GiB buffer is
    overwritten between steps (evicting the L2s and the 256 MB last-level cache, so the
    indices, Q and the gathered rows all come from HBM), and a pair of HIP events on the
    launch stream brackets each step alone (the flush runs before the first event)."""
    s_q = layers[0].inp.s_q
    scale = layers[0].inp.scale
    o_acc = torch.empty((S, s_q, 64, 512), device="cuda") if S > 1 else None
    lse_acc = torch.empty((S, s_q, 64), device="cuda") if S > 1 else None
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")

    def step(L):
        smla.sparse_mla_decode(L.q, L.kv, L.indices, S, scale, kv_scale=L.kv_scale, sink=L.sink, o_accum=o_acc,
                               lse_accum=lse_acc, out=L.out, out_scale=L.out_scale)

    for L in layers:
        step(L)
    stream = torch.cuda.current_stream()
    evs = []
    for i in range(steps):
        flush.fill_(float(i & 7))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(layers[i % len(layers)])
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del flush
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))


def time_cold_kernel(layers, S, steps, torch, smla, flush_bytes=1 << 30):
    """Median duration of the attention kernel alone with every cache flushed before it
    (as time_cold, with partial-only calls; the direct path when S == 1)."""
    s_q = layers[0].inp.s_q
    scale = layers[0].inp.scale
    o_acc = torch.empty((S, s_q, 64, 512), device="cuda") if S > 1 else None
    lse_acc = torch.empty((S, s_q, 64), device="cuda") if S > 1 else None
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")

    def call(L):
        smla.sparse_mla_decode(L.q, L.kv, L.indices, S, scale, kv_scale=L.kv_scale, sink=L.sink, o_accum=o_acc,
                               lse_accum=lse_acc, out=None if S > 1 else L.out,
                               out_scale=None if S > 1 else L.out_scale)

    for L in layers:
        call(L)
    stream = torch.cuda.current_stream()
    evs = []
    for i in range(steps):
        flush.fill_(float(i & 7))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call(layers[i % len(layers)])
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del flush
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))


def sleep_cycles_for(ms, torch):
    """torch.cuda._sleep argument that keeps the GPU busy about `ms` milliseconds."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 1_000_000
    e0.record()
    torch.cuda._sleep(cyc)
    e1.record()
    torch.cuda.synchronize()
    per_ms = cyc / max(e0.elapsed_time(e1), 1e-3)
    return int(per_ms * ms)


def kernel_durations(layers, S, reps, torch, smla):
    """Mean duration (us) of the attention kernel and of the combine, from HIP events on
    the stream they are launched on.  Each figure is a batch of `reps` back-to-back calls
    bracketed by one event pair; a GPU sleep queued first keeps the stream backed up so
    the launches run without host gaps, and `reps` untimed calls run between the sleep
    and the batch, so that it is timed at the clock the GPU holds under sustained load
    (for the first millisecond or so after idling it runs faster: at s_q = 384 a kernel
    takes about 71 us there and 80-85 us once the load has lasted).  The attention kernel is timed alone (partial-only
    calls); the combine as the difference between whole steps and partial-only calls, so
    it is the combine the step runs (an FP8 output's included: its counters are seeded by
    the attention kernel).  S == 1 times the direct path (one kernel per step)."""
    s_q = layers[0].inp.s_q
    scale = layers[0].inp.scale
    stream = torch.cuda.current_stream()
    o_acc = torch.empty((S, s_q, 64, 512), device="cuda") if S > 1 else None
    lse_acc = torch.empty((S, s_q, 64), device="cuda") if S > 1 else None

    def batch(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cyc = sleep_cycles_for(5 + reps * 0.2, torch)
        torch.cuda.synchronize()
        torch.cuda._sleep(cyc)
        for i in range(reps):             # sustained load before the timed calls
            fn(layers[i % len(layers)])
        e0.record(stream)
        for i in range(reps):
            fn(layers[i % len(layers)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    if S == 1:
        main = batch(lambda L: smla.sparse_mla_decode(L.q, L.kv, L.indices, 1, scale, kv_scale=L.kv_scale,
                                                      sink=L.sink, out=L.out, out_scale=L.out_scale))
        return main, 0.0
    main = batch(lambda L: smla.sparse_mla_decode(L.q, L.kv, L.indices, S, scale, kv_scale=L.kv_scale,
                                                  sink=L.sink, o_accum=o_acc, lse_accum=lse_acc))
    step = batch(lambda L: smla.sparse_mla_decode(L.q, L.kv, L.indices, S, scale, kv_scale=L.kv_scale,
                                                  sink=L.sink, o_accum=o_acc, lse_accum=lse_acc, out=L.out,
                                                  out_scale=L.out_scale))
    return main, max(step - main, 0.0)


def traffic_for(S):
    """HBM bytes per launch of the attention kernel from the committed PMC summary,
    or None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_hash() or t.get("num_splits") != S:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(layer, seconds):
    """The float64 oracle (oracle.attend + apply_sink) on the same inputs, on the host
    cores: the median step of `seconds` of repeats with the BLAS pool at its default
    size, then of a third as long with one thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    inp = layer.inp

    class Pool:
        def __getitem__(self, rows):
            from sparse_mla_decode_top_amd.workloads import bf16_bits_to_f32
            return bf16_bits_to_f32(inp.kv_bits[rows])

    q64 = inp.q.astype(np.float64)
    sink = inp.sink.astype(np.float64)

    def median_step(sec):
        times = []
        t_end = time.perf_counter() + sec
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            O, L = oracle.attend(q64, Pool(), inp.indices, inp.n_pool, inp.scale)
            oracle.apply_sink(O, L, sink)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    med, n = median_step(seconds)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        med1, n1 = median_step(seconds / 3)
    return {"value": round(med * 1e6, 1), "unit": "us/step", "cores": int(threads),
            "kind": "oracle",
            "sample": f"whole step ({inp.s_q} token x 64 heads x 640 slots, float64), median of "
                      f"{n} runs in {seconds:.0f} s on {_CORES} host cores",
            "value_1_thread": round(med1 * 1e6, 1),
            "sample_1_thread": f"the same step with the BLAS pool limited to 1 thread, median of {n1} runs"}


def measure(name, S_arg, steps, warmup, reps, torch, smla, W):
    s_q, n_pool, dtype, S_fixed = WORKLOADS[name]
    S = S_arg or S_fixed or smla.smla_choose_num_splits(s_q, 64, 640, 256)
    layers = build_layers(s_q, n_pool, torch, W, dtype=dtype)
    us, ev_us, k, w = time_steps(layers, S, steps, warmup, torch, smla)
    main_us, comb_us = kernel_durations(layers, S, reps, torch, smla)
    cold_us = time_cold(layers, S, max(20, steps // 4), torch, smla)
    cold_main_us = time_cold_kernel(layers, S, max(20, steps // 4), torch, smla)
    step_bytes = STEP_BYTES_PER_TOKEN if dtype == "bf16" else MAIN_BYTES_PER_TOKEN_FP8 + 64 * 512 + 4
    step_gbs = step_bytes * s_q / (ev_us * 1e-6) / 1e9
    return dict(name=name, s_q=s_q, n_pool=n_pool, S=S, us=us, ev_us=ev_us, steps=k, warmup=w,
                main_us=main_us, comb_us=comb_us, step_tbps=step_gbs / 1e3, cold_us=cold_us,
                cold_main_us=cold_main_us,
                layers=len(layers)), layers


def kernel_bytes(name, S):
    """Algorithmic bytes per token of the attention kernel: the gathered rows, Q and the
    indices, plus the output when the kernel writes it (the direct path, S = 1)."""
    pool = WORKLOADS[name][2]
    b = MAIN_BYTES_PER_TOKEN if pool == "bf16" else MAIN_BYTES_PER_TOKEN_FP8
    if S == 1:
        b += OUT_BYTES if pool == "bf16" else 64 * 512 + 4
    return b


def prefill_work(name, W):
    """Algorithmic flops and HBM bytes of one prefill step of a workload: 4 * 128
    flops (QK^T and PV) per visible (row, key) pair and query head; bytes = the e4m3
    Q, K, V read once plus the bf16 output (split partials are overhead, not counted)."""
    B, hq, hk, sq, skv, causal = W.PREFILL_WORKLOADS[name]
    pairs = 0
    for i in range(sq):
        pairs += min(skv, max(0, i + skv - sq + 1)) if causal else skv
    flops = 4 * 128 * pairs * hq * B
    nbytes = B * (sq * hq * 128 + 2 * skv * hk * 128 + sq * hq * 128 * 2)
    return flops, nbytes


def measure_prefill(name, steps, warmup, reps, torch, smla, W):
    """Graph-replayed step (attention + combine), the attention kernel alone (event
    batch), and the cold step, for one prefill workload."""
    B, hq, hk, sq, skv, causal = W.PREFILL_WORKLOADS[name]
    inp = W.make_prefill_inputs(B, hq, hk, sq, skv, 7, causal=causal)
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, k, v, lq, lk, sink = c(inp.q_codes), c(inp.k_codes), c(inp.v_codes), c(inp.seqlen_q), c(inp.seqlen_kv), \
        c(inp.sink)
    S = smla.smla_prefill_choose_splits(B, sq, skv, hq, hk, 256)
    o_part = torch.empty((S, B, sq, hq, 128), device="cuda") if S > 1 else None
    lse_part = torch.empty((S, B, sq, hq), device="cuda") if S > 1 else None
    out = torch.empty((B, sq, hq, 128), device="cuda", dtype=torch.bfloat16)
    amax = torch.empty((1,), device="cuda")

    def step(with_out=True):
        smla.sdpa_fp8_prefill(q, k, v, lq, lk, S, inp.scale, inp.descale_q, inp.descale_k, inp.descale_v,
                              causal=causal, sink=sink, o_part=o_part, lse_part=lse_part,
                              out=out if (with_out or S == 1) else None, amax_out=amax)

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    per = GRAPH_STEPS // 4            # steps a graph (the graph launch cost spread as in time_steps)

    def capture(k):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(k):
                step()
        return g

    g_full = capture(per)
    g_rem = {r: capture(r) for r in {warmup % per, steps % per} if r}

    def replay(k):
        for _ in range(k // per):
            g_full.replay()
        if k % per:
            g_rem[k % per].replay()

    replay(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    replay(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / steps

    def batch(fn):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cyc = sleep_cycles_for(5 + reps * 0.2, torch)
        torch.cuda.synchronize()
        torch.cuda._sleep(cyc)
        for _ in range(reps):             # sustained load before the timed calls (as kernel_durations)
            fn()
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / reps

    main_us = batch(lambda: step(with_out=False))
    full_us = batch(step)
    flush = torch.empty((1 << 30) // 4, dtype=torch.float32, device="cuda")
    evs = []
    for i in range(max(10, steps // 4)):
        flush.fill_(float(i & 7))
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        step()
        a1.record(stream)
        evs.append((a0, a1))
    torch.cuda.synchronize()
    del flush
    cold_us = float(np.median([x.elapsed_time(y) * 1e3 for x, y in evs]))
    flops, nbytes = prefill_work(name, W)
    return {"batch": B, "h_q": hq, "h_kv": hk, "s_q": sq, "s_kv": skv, "causal": causal, "num_splits": S,
            "us_per_step": round(step_us, 2), "cold_us_per_step": round(cold_us, 2),
            "attention_kernel_us": round(main_us, 2), "combine_us": round(max(full_us - main_us, 0.0), 2),
            "algorithmic_tflops": round(flops / (main_us * 1e-6) / 1e12, 1),
            "kernel_mfma_frac": round(flops / (main_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "step_tflops": round(flops / (step_us * 1e-6) / 1e12, 1),
            "kernel_hbm_frac": round(nbytes / (main_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "flops_per_step": flops, "bytes_per_step": nbytes}


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def summarize_kernel_stats(directory):
    rows = _csv_rows(directory, "kernel_stats.csv")
    print(f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for r in rows:
        print(f"{r['Name'][:64]:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.3f} "
              f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f}")
    # The dispatches of the event-timed batches (kernel_durations): a GPU sleep, then
    # one call of the library repeated back to back (one or two kernels per call).
    # Their mean trace duration is the like-for-like counterpart of the HIP-event figure.
    import re
    trace = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))

    def short(name):
        m = re.search(r"::(\w+)<", name)
        return m.group(1) if m else name[:40]

    print("\ndispatches of the event-timed batches (>= 20 repeats of one call's launches after the GPU sleep):")
    print(f"{'kernel':64s} {'batches':>7s} {'calls':>6s} {'avg_us':>9s}")
    agg = {}
    per_call = []
    i = 0
    while i < len(trace):
        if "spin_kernel" not in trace[i]["Kernel_Name"]:
            i += 1
            continue
        # the call's kernels: the launches up to the first repeated name
        period = []
        for r in trace[i + 1:]:
            if "smla::" not in r["Kernel_Name"] or r["Kernel_Name"] in period:
                break
            period.append(r["Kernel_Name"])
        j = i + 1
        while period and j < len(trace) and trace[j]["Kernel_Name"] == period[(j - i - 1) % len(period)]:
            j += 1
        calls = (j - i - 1) // len(period) if period else 0
        if calls >= 20:
            run = trace[i + 1:i + 1 + calls * len(period)]
            tot = 0
            for r in run:
                a = agg.setdefault(r["Kernel_Name"], [0, 0, 0])
                a[1] += 1
                d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                a[2] += d
                tot += d
            for n in period:
                agg[n][0] += 1
            per_call.append((" + ".join(short(n) for n in period), calls, tot / calls / 1e3))
        i = max(j, i + 1)
    for k, (nb, nc, ns) in agg.items():
        print(f"{k[:64]:64s} {nb:7d} {nc:6d} {ns / nc / 1e3:9.3f}")
    for label, calls, us in per_call:
        print(f"batch of {calls} calls ({label}): kernel time per call {us:.3f} us")
    if not per_call:
        print("(none: no batch repeats a call 20 times; the averages above are over all calls)")


def _counter_per_dispatch(directory, counter):
    """{kernel name: mean counter value per dispatch} from a rocprofv3 --pmc run."""
    tot, disp = {}, {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
        disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def hbm_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, scaled by what the
    same counters read for a plain copy of 256 MiB (read and written once)."""
    copy_kib = (256 << 20) / 1024.0

    def pick(d, key):
        hits = [v for k, v in d.items() if key in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {sorted(d)}")
        return hits[0]

    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    f_copy = pick(_counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE"), "copyBuffer")
    w_copy = pick(_counter_per_dispatch(copy_write_dir, "WRITE_SIZE"), "copyBuffer")
    rf, wf = copy_kib / f_copy, copy_kib / w_copy
    print(f"copy calibration: 256 MiB copy reads FETCH_SIZE {f_copy:.1f} KiB -> read factor {rf:.3f}; "
          f"WRITE_SIZE {w_copy:.1f} KiB -> write factor {wf:.3f}")
    print(f"{'kernel':64s} {'FETCH_KiB':>10s} {'WRITE_KiB':>10s} {'HBM_bytes':>12s}")
    for k in sorted(set(fetch) | set(write)):
        b = (fetch.get(k, 0.0) * rf + write.get(k, 0.0) * wf) * 1024
        print(f"{k[:64]:64s} {fetch.get(k, 0.0):10.1f} {write.get(k, 0.0):10.1f} {b:12.0f}")
    kf, kw = pick(fetch, "decode_kernel"), pick(write, "decode_kernel")
    rec = {"kernel": kernel_label(WORKLOADS["single"][0], _single_splits(), "bf16"), "workload": "single",
           "num_splits": _single_splits(),
           "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1),
           "read_factor": round(rf, 4), "write_factor": round(wf, 4),
           "hbm_bytes_per_launch": int(round((kf * rf + kw * wf) * 1024)),
           "kernel_source_sha256": source_hash()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def pmc_summary(dirs):
    """Per kernel and counter: the mean over dispatches of the counter summed (and maxed)
    over its hardware instances.  For the attention kernel also: the MFMA busy share
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) and the executed bf16 and f16 MFMA
    flops SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F16 x 512."""
    per = {}                       # (kernel, counter) -> {dispatch: [values]}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            key = (r["Kernel_Name"], r["Counter_Name"])
            per.setdefault(key, {}).setdefault((d, r["Dispatch_Id"]), []).append(float(r["Counter_Value"]))
    print(f"{'kernel':56s} {'counter':32s} {'dispatches':>10s} {'sum/dispatch':>16s} {'max/dispatch':>16s}")
    stats = {}
    for (k, c), disp in sorted(per.items()):
        sums = [sum(v) for v in disp.values()]
        maxs = [max(v) for v in disp.values()]
        stats[(k, c)] = (np.mean(sums), np.mean(maxs))
        print(f"{k[:56]:56s} {c:32s} {len(disp):10d} {np.mean(sums):16.1f} {np.mean(maxs):16.1f}")
    # GRBM_GUI_ACTIVE comes summed over the 8 XCDs: a dispatch's active cycles are a
    # eighth of it (the MFMA loop probe then reads ~96% busy, as a pure MFMA loop should).
    for k in sorted({k for k, _ in stats if any(n in k for n in ("decode_kernel", "mfma_loop", "prefill_kernel"))}):
        busy = stats.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"))
        active = stats.get((k, "GRBM_GUI_ACTIVE"))
        mops = stats.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        mops16 = stats.get((k, "SQ_INSTS_VALU_MFMA_MOPS_F16"))
        if busy and active:
            cyc = active[0] / 8
            print(f"{k[:56]}: MFMA busy {busy[0]:.0f} SIMD-cycles over {cyc:.0f} active cycles x 1024 SIMDs "
                  f"= {100.0 * busy[0] / (cyc * 1024):.1f}%")
        if mops:
            print(f"{k[:56]}: executed bf16 MFMA flops per dispatch {mops[0] * 512:.4g}")
        if mops16:
            print(f"{k[:56]}: executed f16 MFMA flops per dispatch {mops16[0] * 512:.4g}")


def kernel_label(s_q, S, pool, cus=256):
    """Which attention kernel(s) a launch runs (mirrors sparse_mla_decode's choice for 64
    heads): the head-tile kernel at 4, 8 or 16 parts, the head-half kernel at 2, the paired
    8-wave kernel at one part; a last round that would fill at most half of the CUs takes
    two head halves in the same launch (the mixed kernel)."""
    jobs = s_q * S
    cs = 16 if 16 * jobs <= cus else 8 if 8 * jobs <= cus else 4 if 4 * jobs <= cus else 2 if 2 * jobs <= cus else 1
    mode = "partial" if S > 1 else "direct"

    def one(c):
        if c in (4, 8, 16):
            cols = {4: "", 8: " x column halves", 16: " x column quarters"}[c]
            return f"decode_kernel4t<{pool} pool, {mode}, {c} parts: head tiles{cols}>"
        if c == 2:
            return f"decode_kernel8h<{pool} pool, {mode}, 2 head halves>"
        return f"decode_kernel8p<{pool} pool, {mode}, 1 column part>"

    tail = jobs % cus
    if cs == 1 and jobs > cus and 0 < tail and 2 * tail <= cus and (jobs - tail) % 8 == 0:
        return (f"decode_kernel8m<{pool} pool, {mode}: decode_kernel8p's body over {jobs - tail} jobs, "
                f"decode_kernel8h's in 2 head halves over the last {tail}>")
    return one(cs)


def _single_splits():
    from sparse_mla_decode_top_amd import binding
    return binding.smla_choose_num_splits(WORKLOADS["single"][0], 64, 640, 256)


def measured_peaks(torch):
    """Peak denominators measured on this GPU, reported beside the published ones:
    HBM read (1 GiB streamed in 16-byte loads), HBM copy (1 GiB read + 1 GiB
    written), and the bf16 matrix-core rate of an MFMA issue loop (both probes in
    libsmla_peak.so)."""
    import ctypes
    n = 1 << 28                                     # 1 GiB of float32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    peak = ctypes.CDLL(os.path.join(ROOT, "sparse_mla_decode_top_amd", "libsmla_peak.so"))
    peak.smla_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    peak.smla_peak_mfma_bf16.restype = ctypes.c_int
    peak.smla_peak_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    peak.smla_peak_mfma_flops.restype = ctypes.c_double
    peak.smla_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    peak.smla_peak_hbm_read.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    rblocks = 4096
    words = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")

    def read():
        if peak.smla_peak_hbm_read(a.data_ptr(), n * 4, rblocks, words.data_ptr(), stream) != 0:
            raise RuntimeError("smla_peak_hbm_read failed")

    t_read = timed(read, 10)
    t_copy = timed(lambda: b.copy_(a), 10)
    del a, b, words
    torch.cuda.empty_cache()
    blocks, iters = 1024, 2000
    out = torch.empty(blocks * 256, device="cuda")

    def mfma():
        if peak.smla_peak_mfma_bf16(blocks, iters, out.data_ptr(), stream) != 0:
            raise RuntimeError("smla_peak_mfma_bf16 failed")

    t_mfma = timed(mfma, 3)
    return {"hbm_read_gbs": round(n * 4 / t_read / 1e9, 1), "hbm_copy_gbs": round(2 * n * 4 / t_copy / 1e9, 1),
            "mfma_bf16_tflops": round(peak.smla_peak_mfma_flops(blocks, iters) / t_mfma / 1e12, 1),
            "published": {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": BF16_PEAK_TFLOPS}}


def copy_only(torch):
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}), flush=True)


def main():
    args = parse_args()
    if args.kernel_stats:
        summarize_kernel_stats(args.kernel_stats)
        return
    if args.hbm_counters:
        hbm_counters(*args.hbm_counters)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the kernels and the launch plan are one GPU's); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    import sparse_mla_decode_top_amd as smla
    from sparse_mla_decode_top_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    smla.load_library()
    if args.copy_only:
        copy_only(torch)
        return
    if args.prefill_only:
        res = {name: measure_prefill(name, args.steps, args.warmup, args.kernel_reps, torch, smla, W)
               for name in W.PREFILL_WORKLOADS}
        print(json.dumps({"prefill": res}), flush=True)
        return

    head, layers = measure(args.workload, args.num_splits, args.steps, args.warmup, args.kernel_reps,
                           torch, smla, W)
    s_q, S = head["s_q"], head["S"]
    log(f"{args.workload}: {head['us']:.2f} us/step (events {head['ev_us']:.2f}), attention kernel "
        f"{head['main_us']:.2f} us, combine {head['comb_us']:.2f} us, cold step {head['cold_us']:.2f} us, S={S}")
    pool_dtype = WORKLOADS[args.workload][2]
    main_bytes = kernel_bytes(args.workload, S) * s_q
    achieved = main_bytes / (head["main_us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(S),
                "kernel": kernel_label(s_q, S, pool_dtype),
                "bytes_per_launch": main_bytes, "mean_launch_us": round(head["main_us"], 3),
                "cache": "warm: back-to-back launches cycling over the layers, whose gathered rows stay in "
                         "the last-level cache at this size; cold_* flush every cache before each launch",
                "cold_launch_us": round(head["cold_main_us"], 3),
                "cold_achieved": round(main_bytes / (head["cold_main_us"] * 1e-6) / 1e9, 1),
                "cold_frac": round(main_bytes / (head["cold_main_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(FLOPS_PER_TOKEN * s_q / (head["main_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 5)}
    peaks = measured_peaks(torch)
    log(f"measured peaks: {peaks}")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host cores")
        cpu = cpu_baseline(layers[0], args.cpu_seconds)
    del layers
    torch.cuda.empty_cache()

    sweep = {}
    if not args.no_sweep:
        for name in ("small6", "small16", "large96", "large384", "fp8_1", "fp8_16"):
            if name == args.workload:
                continue
            r, ls = measure(name, 0, max(20, args.steps // 4), args.warmup, max(20, args.kernel_reps // 4),
                            torch, smla, W)
            del ls
            torch.cuda.empty_cache()
            mb = kernel_bytes(name, r["S"]) * r["s_q"]
            sweep[name] = {"s_q": r["s_q"], "pool": WORKLOADS[name][2], "num_splits": r["S"],
                           "us_per_step": round(r["ev_us"], 2), "cold_us_per_step": round(r["cold_us"], 2),
                           "attention_kernel_us": round(r["main_us"], 2), "combine_us": round(r["comb_us"], 2),
                           "cold_attention_kernel_us": round(r["cold_main_us"], 2),
                           "step_hbm_tbps": round(r["step_tbps"], 3),
                           "kernel_hbm_frac": round(mb / (r["main_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "kernel_mfma_frac": round(FLOPS_PER_TOKEN * r["s_q"] / (r["main_us"] * 1e-6) / 1e12
                                                     / BF16_PEAK_TFLOPS, 4)}
            log(f"{name}: {r['ev_us']:.2f} us/step, kernel {r['main_us']:.2f} us, cold step {r['cold_us']:.2f} us, "
                f"S={r['S']}")
        for name in W.PREFILL_WORKLOADS:
            r = measure_prefill(name, max(20, args.steps // 4), args.warmup, max(20, args.kernel_reps // 4),
                                torch, smla, W)
            torch.cuda.empty_cache()
            sweep[name] = r
            log(f"{name}: {r['us_per_step']:.2f} us/step, kernel {r['attention_kernel_us']:.2f} us "
                f"({r['algorithmic_tflops']} TFLOP/s), S={r['num_splits']}")

    line = {
        "metric": METRIC, "value": round(head["ev_us"], 3), "unit": "us/step", "n_gpus": 1,
        "steps": head["steps"], "warmup": head["warmup"], "ms_per_step": round(head["ev_us"] / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if pool_dtype == "bf16" else "fp8_e4m3 (bf16 MFMA)",
        "data": "synthetic (seeded N(0,1) bf16 pools, uniform unique top-k indices)",
        "config": {"workload": f"{LABELS[args.workload]}: s_q={s_q}, h_q=64, d_qk=576, d_v=512, topk=640, "
                               f"pool {head['n_pool']} {pool_dtype} rows x {head['layers']} layers, sink on, "
                               f"num_splits={S}",
                   "global_batch": s_q, "num_splits": S,
                   "timing": f"exactly {args.warmup} untimed then {args.steps} timed steps, HIP graph replay "
                             f"cycling over the layers, {GRAPH_STEPS} steps a graph; warm: the rows all layers gather stay in the 256 MB "
                             "last-level cache at this size, so value and roofline are warm-cache figures; "
                             "cold_us_per_step flushes every cache before each step"},
        "hbm_tbps": round(head["step_tbps"], 4),
        "cold_us_per_step": round(head["cold_us"], 3),
        "wall_us_per_step": round(head["us"], 3),
        "attention_kernel_us": round(head["main_us"], 3),
        "combine_kernel_us": round(head["comb_us"], 3),
        "roofline": roofline,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "context": {"b200_fused_kernel_us_s_q1": {"unsplit": 26.6, "split8": 14.4, "split16": 14.3}},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
