"""Host-side tests of the C ABI (no GPU): the library loads, exports every
function include/smla.h declares, and its argument checks, split heuristic and
size helper behave as documented.  Pointers handed to smla_validate are plain
integers; the library only tests them for NULL and alignment."""
import ctypes
import os
import re

import pytest

import sparse_mla_decode_top_amd as smla
from sparse_mla_decode_top_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

OK, INVALID, UNSUPPORTED, MISSING_WS, MISALIGNED = 0, 1, 2, 3, 4
A = 0x10000          # a 16-byte aligned stand-in address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof", "defined"})


def test_library_exports_every_declared_function():
    lib = B.load_library()
    names = declared_functions()
    assert set(names) == set(B.SIGNATURES), names
    for n in names:
        assert getattr(lib, n) is not None


def test_struct_layout_matches_header():
    assert ctypes.sizeof(B.SmlaParams) == 48
    assert B.SmlaParams.n_pool.offset == 16 and B.SmlaParams.softmax_scale.offset == 32


def test_status_strings():
    for code, name in B.STATUS_NAMES.items():
        assert smla.smla_status_string(code) == name
    assert smla.smla_status_string(99) == "SMLA_ERR_UNKNOWN"


def test_partial_bytes():
    assert smla.smla_partial_bytes(1, 64, 8) == 8 * 64 * (512 * 4 + 4)
    assert smla.smla_partial_bytes(16, 64, 8) == 16 * 8 * 64 * 2052
    assert smla.smla_partial_bytes(0, 64, 8) == 0
    assert smla.smla_partial_bytes(1, 64, 0) == 0


def test_choose_num_splits_properties():
    for s_q in (1, 2, 6, 16, 96, 127, 128, 384, 1000):
        for topk in (1, 64, 100, 640, 2048):
            s = smla.smla_choose_num_splits(s_q, 64, topk, 256)
            n_blk = -(-topk // 64)
            assert 1 <= s <= max(1, min(n_blk, 64))
            if s > 1:
                assert 2 * s_q * s <= 256      # split jobs keep two column parts in one round
            if s_q > 32:
                assert s == 1
    for s_q, expect in ((1, 10), (4, 8), (6, 5), (8, 4), (16, 4), (17, 2), (32, 2), (33, 1), (64, 1), (96, 1), (384, 1)):
        assert smla.smla_choose_num_splits(s_q, 64, 640, 256) == expect, s_q
    assert smla.smla_choose_num_splits(32, 64, 640, 512) == 4      # scales with the CU count
    assert smla.smla_choose_num_splits(8, 64, 640, 512) == 8
    assert smla.smla_choose_num_splits(1, 64, 64, 256) == 1        # capped at the block count
    assert smla.smla_choose_num_splits(0, 64, 640, 256) == 0
    # deterministic
    assert smla.smla_choose_num_splits(16, 64, 640, 256) == smla.smla_choose_num_splits(16, 64, 640, 256)


def test_prefill_choose_splits_rule():
    """Workgroups of the unsplit prefill launch: batch x 64-row tiles x h_q / HPW (HPW = 2
    when h_q / h_kv is even); S brings them to about two per compute unit, capped at the
    KV blocks and at 16."""
    c = smla.smla_prefill_choose_splits
    assert c(2, 256, 8192, 32, 8, 256) == 4          # 128 workgroups unsplit
    assert c(1, 4096, 4096, 32, 8, 256) == 1         # 1,024 already fill two rounds
    assert c(1, 256, 8192, 6, 2, 256) == 16          # odd ratio: 24 workgroups -> 22, capped at 16
    assert c(1, 64, 8192, 32, 32, 64) == 4           # one query head a KV head: 32 workgroups
    assert c(1, 64, 8192, 32, 16, 64) == 8           # pairs: 16 workgroups
    assert c(1, 64, 100, 2, 1, 256) == 2             # 1 workgroup -> capped at the 2 KV blocks
    assert c(4, 64, 8192, 8, 8, 256) == 16           # 32 workgroups -> 16
    assert c(1, 64, 8192, 64, 1, 256) == 16          # HPW 2: 32 workgroups -> 16
    assert c(1, 64, 8192, 64, 1, 64) == 4            # scales with the CU count
    assert c(1, 256, 8192, 6, 4, 256) == 0           # h_q not a multiple of h_kv
    assert c(0, 256, 8192, 32, 8, 256) == 0
    assert c(1, 256, 8192, 32, 0, 256) == 0


def _p(**kw):
    base = dict(s_q=2, h_q=64, topk=640, n_pool=1000, kv_row_stride=576, softmax_scale=1 / 24,
                kv_dtype=B.KV_BF16, out_dtype=B.OUT_BF16)
    base.update(kw)
    return B.make_params(**base)


def _v(params, **kw):
    args = dict(q=A, kv_pool=A, kv_scale=None, indices=A, num_splits=1, o_accum=None, lse_accum=None,
                out=A, out_scale=None)
    args.update(kw)
    return B.smla_validate(params, **args)


def test_validate_accepts_the_documented_modes():
    assert _v(_p()) == OK                                                 # direct path
    assert _v(_p(), num_splits=8, o_accum=A, lse_accum=A) == OK           # split + combine
    assert _v(_p(), num_splits=8, o_accum=A, lse_accum=A, out=None) == OK  # partial only
    assert _v(_p(), num_splits=1, o_accum=A, lse_accum=A) == OK           # S=1 through partials
    assert _v(_p(h_q=16)) == OK and _v(_p(h_q=32)) == OK
    assert _v(_p(kv_dtype=B.KV_FP8_E4M3), kv_scale=A) == OK
    assert _v(_p(out_dtype=B.OUT_FP8_E4M3), out_scale=A) == OK
    assert _v(_p(kv_row_stride=640)) == OK


@pytest.mark.parametrize("kw,params,expect", [
    ({}, dict(s_q=0), INVALID),
    ({}, dict(topk=0), INVALID),
    ({}, dict(n_pool=0), INVALID),
    ({}, dict(h_q=48), UNSUPPORTED),
    ({}, dict(h_q=128), UNSUPPORTED),
    ({}, dict(split_block=32), UNSUPPORTED),
    ({}, dict(kv_dtype=7), INVALID),
    ({}, dict(out_dtype=9), INVALID),
    ({}, dict(softmax_scale=float("nan")), INVALID),
    ({}, dict(kv_row_stride=512), INVALID),
    ({}, dict(kv_row_stride=580), MISALIGNED),                 # 1160 bytes: not 16-byte aligned
    (dict(num_splits=0), {}, INVALID),
    (dict(num_splits=65, o_accum=A, lse_accum=A), {}, UNSUPPORTED),
    (dict(num_splits=4), {}, MISSING_WS),                      # split without partial buffers
    (dict(num_splits=4, o_accum=A), {}, MISSING_WS),
    (dict(num_splits=1, lse_accum=A), {}, MISSING_WS),
    (dict(out=None), {}, INVALID),                             # direct path with no output
    (dict(q=None), {}, INVALID),
    (dict(kv_pool=None), {}, INVALID),
    (dict(indices=None), {}, INVALID),
    (dict(q=A + 8), {}, MISALIGNED),
    (dict(kv_pool=A + 4), {}, MISALIGNED),
    (dict(indices=A + 2), {}, MISALIGNED),
    (dict(out=A + 8), {}, MISALIGNED),
    (dict(num_splits=2, o_accum=A + 4, lse_accum=A), {}, MISALIGNED),
    ({}, dict(kv_dtype=1), INVALID),                           # FP8 pool without row scales
    ({}, dict(out_dtype=2), INVALID),                          # FP8 output without out_scale
])
def test_validate_rejects(kw, params, expect):
    assert _v(_p(**params), **kw) == expect


def test_fp8_row_stride_is_in_bytes():
    assert _v(_p(kv_dtype=B.KV_FP8_E4M3, kv_row_stride=576), kv_scale=A) == OK
    assert _v(_p(kv_dtype=B.KV_FP8_E4M3, kv_row_stride=584), kv_scale=A) == MISALIGNED
    assert _v(_p(kv_dtype=B.KV_FP8_E4M3, kv_row_stride=592), kv_scale=A) == OK


def test_null_params_rejected():
    lib = B.load_library()
    assert lib.smla_validate(None, A, A, None, A, 1, None, None, A, None) == INVALID
    assert lib.combine_splits(None, 1, A, A, None, A, None, None, None) == INVALID


def test_combine_rejects_before_launch():
    lib = B.load_library()
    p = _p()
    assert lib.combine_splits(ctypes.byref(p), 2, None, A, None, A, None, None, None) == MISSING_WS
    assert lib.combine_splits(ctypes.byref(p), 2, A, A, None, None, None, None, None) == INVALID
    assert lib.combine_splits(ctypes.byref(p), 0, A, A, None, A, None, None, None) == INVALID
    assert lib.combine_splits(ctypes.byref(p), 2, A + 4, A, None, A, None, None, None) == MISALIGNED
    p8 = _p(out_dtype=B.OUT_FP8_E4M3)
    assert lib.combine_splits(ctypes.byref(p8), 2, A, A, None, A, None, None, None) == INVALID


def test_decode_rejects_before_launch():
    """Argument errors come back as status codes before anything touches the GPU."""
    lib = B.load_library()
    p = _p()
    st = lib.sparse_mla_decode(ctypes.byref(p), A, A, None, A, 4, None, None, None, A, None, None, None)
    assert st == MISSING_WS
    st = lib.sparse_mla_decode(ctypes.byref(_p(h_q=8)), A, A, None, A, 1, None, None, None, A, None, None, None)
    assert st == UNSUPPORTED


@pytest.mark.parametrize("scale,dq,dk,expect", [
    (0.0, 1.0, 1.0, INVALID),              # the score scale must be positive
    (-0.088, 1.0, 1.0, INVALID),
    (0.088, -1.0, 1.0, INVALID),
    (1e-20, 1e-20, 1.0, INVALID),          # 1e-40: below 2^-100
    (float("inf"), 1.0, 1.0, INVALID),
    (0.088, 1.0, float("nan"), INVALID),
    (0.088, -1.0, -1.0, OK),               # a positive product is accepted
])
def test_prefill_score_scale_checked_before_launch(scale, dq, dk, expect):
    """sdpa_fp8_prefill rejects a score scale softmax_scale * descale_q * descale_k that is not
    positive and at least 2^-100 before anything touches the GPU.  An accepted scale is shown with
    split_kv = 2 and no partials, which the next check rejects, still before any launch."""
    lib = B.load_library()
    p = B.make_prefill_params(1, 8, 8, 64, 64, scale, dq, dk)
    st = lib.sdpa_fp8_prefill(ctypes.byref(p), A, A, A, A, A, 2, None, None, None, A, None, None, None)
    assert st == (MISSING_WS if expect == OK else expect)


def test_noalloc_rejects_before_launch():
    """sparse_mla_decode_noalloc: a missing output, a bad shape and partials larger than
    its scratch come back as status codes before anything touches the GPU."""
    lib = B.load_library()
    p = _p()
    args = (A, A, None, A)
    assert lib.sparse_mla_decode_noalloc(ctypes.byref(p), *args, 8, None, None, None, None, None) == INVALID
    assert lib.sparse_mla_decode_noalloc(ctypes.byref(_p(h_q=8)), *args, 8, None, A, None, None, None) == UNSUPPORTED
    assert lib.sparse_mla_decode_noalloc(ctypes.byref(p), *args, 0, None, A, None, None, None) == INVALID
    big = _p(s_q=6)
    assert smla.smla_partial_bytes(6, 64, 64) > B.NOALLOC_SCRATCH_BYTES
    assert lib.sparse_mla_decode_noalloc(ctypes.byref(big), *args, 64, None, A, None, None, None) == 6


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    assert "#define SMLA_NOALLOC_SCRATCH_BYTES (32u << 20)" in text
    assert B.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_peak_probe_exports_its_header():
    """libsmla_peak.so (bench.py's matrix-core probe) exports what include/smla_peak.h declares."""
    text = open(os.path.join(ROOT, "include", "smla_peak.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text))
    assert names == {"smla_peak_mfma_bf16", "smla_peak_mfma_flops", "smla_peak_hbm_read"}
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mla_decode_top_amd", "libsmla_peak.so"))
    lib.smla_peak_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.smla_peak_mfma_flops.restype = ctypes.c_double
    assert lib.smla_peak_mfma_flops(2, 3) == 2 * 4 * 3 * 16 * (16 * 16 * 32 * 2)
    lib.smla_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.smla_peak_mfma_bf16(0, 1, A, None) == 1          # rejected before any launch
    assert lib.smla_peak_mfma_bf16(1, 1, None, None) == 1
    lib.smla_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    assert lib.smla_peak_hbm_read(A + 8, 1 << 20, 4, A, None) == 1     # misaligned
    assert lib.smla_peak_hbm_read(A, 8, 4, A, None) == 1               # shorter than one load
