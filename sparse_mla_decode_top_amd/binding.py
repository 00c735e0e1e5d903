"""ctypes binding to libsmla.so, the C-ABI declared in include/smla.h.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Tensors are PyTorch CUDA tensors (torch is used for device memory and
the current stream); their ``data_ptr()`` is handed to the library.  The
library must be built (``python -m sparse_mla_decode_top_amd.build``); if it is
missing every call raises ``SmlaError`` -- there is no CPU fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsmla.so"

KV_BF16, KV_FP8_E4M3 = 0, 1
OUT_BF16, OUT_FP32, OUT_FP8_E4M3 = 0, 1, 2
D_QK, D_V, SPLIT_BLOCK, MAX_SPLITS = 576, 512, 64, 64
NOALLOC_SCRATCH_BYTES = 32 << 20

STATUS_NAMES = {
    0: "SMLA_OK", 1: "SMLA_ERR_INVALID_ARG", 2: "SMLA_ERR_UNSUPPORTED",
    3: "SMLA_ERR_MISSING_WORKSPACE", 4: "SMLA_ERR_MISALIGNED", 5: "SMLA_ERR_HIP",
    6: "SMLA_ERR_SCRATCH_TOO_SMALL",
}


class SmlaError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class SmlaParams(ctypes.Structure):
    _fields_ = [
        ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("split_block", ctypes.c_int32), ("n_pool", ctypes.c_int64),
        ("kv_row_stride", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
        ("kv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


class SmlaPrefillParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_s_q", ctypes.c_int32), ("max_s_kv", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("q_tile", ctypes.c_int32), ("kv_block", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float),
        ("descale_v", ctypes.c_float), ("out_dtype", ctypes.c_int32),
    ]


_lib = None
_vp = ctypes.c_void_p

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "sparse_mla_decode": (ctypes.c_int, [ctypes.POINTER(SmlaParams), _vp, _vp, _vp, _vp, ctypes.c_int32,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sparse_mla_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(SmlaParams), _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                 _vp, _vp, _vp, _vp, _vp]),
    "combine_splits": (ctypes.c_int, [ctypes.POINTER(SmlaParams), ctypes.c_int32, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp]),
    "smla_choose_num_splits": (ctypes.c_int32, [ctypes.c_int32] * 4),
    "smla_partial_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "smla_validate": (ctypes.c_int, [ctypes.POINTER(SmlaParams), _vp, _vp, _vp, _vp, ctypes.c_int32,
                                     _vp, _vp, _vp, _vp]),
    "smla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sdpa_fp8_prefill": (ctypes.c_int, [ctypes.POINTER(SmlaPrefillParams), _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "smla_prefill_partial_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 4),
    "smla_prefill_choose_splits": (ctypes.c_int32, [ctypes.c_int32] * 6),
}


def library_path():
    return os.environ.get("SMLA_LIBRARY", os.path.join(HERE, _LIB_NAME))


def load_library():
    """Load libsmla.so once; raise SmlaError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise SmlaError(f"{path} is missing: build it with `python -m sparse_mla_decode_top_amd.build` "
                        "(the decode has no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def smla_status_string(status):
    return load_library().smla_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise SmlaError(f"{what} failed: {smla_status_string(status)}", status)


def smla_choose_num_splits(s_q, h_q, topk, num_cus=256):
    return int(load_library().smla_choose_num_splits(s_q, h_q, topk, num_cus))


def smla_partial_bytes(s_q, h_q, num_splits):
    return int(load_library().smla_partial_bytes(s_q, h_q, num_splits))


def make_params(s_q, h_q, topk, n_pool, kv_row_stride, softmax_scale, kv_dtype=KV_BF16,
                out_dtype=OUT_BF16, split_block=SPLIT_BLOCK):
    return SmlaParams(s_q=s_q, h_q=h_q, topk=topk, split_block=split_block, n_pool=n_pool,
                      kv_row_stride=kv_row_stride, softmax_scale=softmax_scale,
                      kv_dtype=kv_dtype, out_dtype=out_dtype)


def smla_validate(params, q=None, kv_pool=None, kv_scale=None, indices=None, num_splits=1,
                  o_accum=None, lse_accum=None, out=None, out_scale=None):
    """Host-side argument check; pointers may be plain integers (never dereferenced)."""
    return int(load_library().smla_validate(ctypes.byref(params), q, kv_pool, kv_scale, indices,
                                            num_splits, o_accum, lse_accum, out, out_scale))


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------
def _ptr(t):
    return None if t is None else t.data_ptr()


def _out_dtype_of(out, out_dtype):
    import torch
    if out_dtype is not None:
        return out_dtype
    if out is None:
        return OUT_BF16
    if out.dtype == torch.bfloat16:
        return OUT_BF16
    if out.dtype == torch.float32:
        return OUT_FP32
    if out.dtype in (torch.uint8, torch.float8_e4m3fn):
        return OUT_FP8_E4M3
    raise SmlaError(f"unsupported output dtype {out.dtype}")


def _need(t, name, numel, dtypes, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise SmlaError(f"{name} must be a CUDA tensor on {device}")
    if not t.is_contiguous():
        raise SmlaError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise SmlaError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < numel:
        raise SmlaError(f"{name} holds {t.numel()} elements, needs {numel}")


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def sparse_mla_decode(q, kv_pool, indices, num_splits, softmax_scale, kv_scale=None, sink=None,
                      o_accum=None, lse_accum=None, out=None, out_scale=None, lse_out=None,
                      out_dtype=None, stream=None):
    """Run the decode step through the C ABI (see include/smla.h for the modes).

    q [s_q, h_q, 576] bf16; kv_pool [n_pool, row_stride] bf16, or uint8 e4m3 codes with
    kv_scale [n_pool] f32; indices [s_q, topk] int32.  The output dtype follows `out`
    (bf16 / float32 / uint8 codes) unless `out_dtype` is given.
    """
    import torch
    lib = load_library()
    s_q, h_q, dqk = q.shape
    topk = indices.shape[1]
    n_pool, row_stride = kv_pool.shape
    kv_dtype = KV_FP8_E4M3 if kv_pool.dtype in (torch.uint8, torch.float8_e4m3fn) else KV_BF16
    od = _out_dtype_of(out, out_dtype)
    dev = q.device
    if dqk != D_QK or indices.shape[0] != s_q:
        raise SmlaError("shape mismatch between q and indices")
    _need(q, "q", s_q * h_q * D_QK, (torch.bfloat16,), dev)
    _need(kv_pool, "kv_pool", n_pool * row_stride, (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev)
    _need(kv_scale, "kv_scale", n_pool, (torch.float32,), dev)
    _need(indices, "indices", s_q * topk, (torch.int32,), dev)
    _need(sink, "sink", h_q, (torch.float32,), dev)
    _need(o_accum, "o_accum", num_splits * s_q * h_q * D_V, (torch.float32,), dev)
    _need(lse_accum, "lse_accum", num_splits * s_q * h_q, (torch.float32,), dev)
    out_types = {OUT_BF16: (torch.bfloat16,), OUT_FP32: (torch.float32,),
                 OUT_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}[od]
    _need(out, "out", s_q * h_q * D_V, out_types, dev)
    _need(out_scale, "out_scale", s_q, (torch.float32,), dev)
    _need(lse_out, "lse_out", s_q * h_q, (torch.float32,), dev)
    p = make_params(s_q, h_q, topk, n_pool, row_stride, softmax_scale, kv_dtype, od)
    st = lib.sparse_mla_decode(ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(kv_scale), _ptr(indices),
                               int(num_splits), _ptr(sink), _ptr(o_accum), _ptr(lse_accum), _ptr(out),
                               _ptr(out_scale), _ptr(lse_out), _stream_handle(stream, dev))
    _check(st, "sparse_mla_decode")


def sparse_mla_decode_noalloc(q, kv_pool, indices, num_splits, softmax_scale, out, kv_scale=None, sink=None,
                              out_scale=None, lse_out=None, out_dtype=None, stream=None):
    """The decode step with its split partials in the library's own device scratch
    (include/smla.h, sparse_mla_decode_noalloc): no workspace arguments, `out` required."""
    import torch
    lib = load_library()
    s_q, h_q, dqk = q.shape
    topk = indices.shape[1]
    n_pool, row_stride = kv_pool.shape
    kv_dtype = KV_FP8_E4M3 if kv_pool.dtype in (torch.uint8, torch.float8_e4m3fn) else KV_BF16
    od = _out_dtype_of(out, out_dtype)
    dev = q.device
    if dqk != D_QK or indices.shape[0] != s_q:
        raise SmlaError("shape mismatch between q and indices")
    _need(q, "q", s_q * h_q * D_QK, (torch.bfloat16,), dev)
    _need(kv_pool, "kv_pool", n_pool * row_stride, (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), dev)
    _need(kv_scale, "kv_scale", n_pool, (torch.float32,), dev)
    _need(indices, "indices", s_q * topk, (torch.int32,), dev)
    _need(sink, "sink", h_q, (torch.float32,), dev)
    out_types = {OUT_BF16: (torch.bfloat16,), OUT_FP32: (torch.float32,),
                 OUT_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}[od]
    _need(out, "out", s_q * h_q * D_V, out_types, dev)
    _need(out_scale, "out_scale", s_q, (torch.float32,), dev)
    _need(lse_out, "lse_out", s_q * h_q, (torch.float32,), dev)
    p = make_params(s_q, h_q, topk, n_pool, row_stride, softmax_scale, kv_dtype, od)
    st = lib.sparse_mla_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(kv_scale), _ptr(indices),
                                       int(num_splits), _ptr(sink), _ptr(out), _ptr(out_scale), _ptr(lse_out),
                                       _stream_handle(stream, dev))
    _check(st, "sparse_mla_decode_noalloc")


def combine_splits(o_accum, lse_accum, num_splits, out, sink=None, out_scale=None, lse_out=None,
                   out_dtype=None, stream=None):
    """Merge split partials o_accum [S, s_q, h_q, 512], lse_accum [S, s_q, h_q] into `out`."""
    import torch
    lib = load_library()
    S, s_q, h_q = lse_accum.shape
    if S != num_splits:
        raise SmlaError("lse_accum's leading dimension must equal num_splits")
    od = _out_dtype_of(out, out_dtype)
    dev = o_accum.device
    _need(o_accum, "o_accum", num_splits * s_q * h_q * D_V, (torch.float32,), dev)
    _need(lse_accum, "lse_accum", num_splits * s_q * h_q, (torch.float32,), dev)
    _need(sink, "sink", h_q, (torch.float32,), dev)
    out_types = {OUT_BF16: (torch.bfloat16,), OUT_FP32: (torch.float32,),
                 OUT_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}[od]
    _need(out, "out", s_q * h_q * D_V, out_types, dev)
    _need(out_scale, "out_scale", s_q, (torch.float32,), dev)
    _need(lse_out, "lse_out", s_q * h_q, (torch.float32,), dev)
    p = make_params(s_q, h_q, 1, 1, D_QK, 1.0, KV_BF16, od)
    st = lib.combine_splits(ctypes.byref(p), int(num_splits), _ptr(o_accum), _ptr(lse_accum), _ptr(sink),
                            _ptr(out), _ptr(out_scale), _ptr(lse_out), _stream_handle(stream, dev))
    _check(st, "combine_splits")


# ---------------------------------------------------------------------------
# split-KV FP8 prefill
# ---------------------------------------------------------------------------
def smla_prefill_partial_bytes(batch, max_s_q, h_q, split_kv):
    return int(load_library().smla_prefill_partial_bytes(batch, max_s_q, h_q, split_kv))


def smla_prefill_choose_splits(batch, max_s_q, max_s_kv, h_q, h_kv, num_cus=256):
    return int(load_library().smla_prefill_choose_splits(batch, max_s_q, max_s_kv, h_q, h_kv, num_cus))


def make_prefill_params(batch, h_q, h_kv, max_s_q, max_s_kv, softmax_scale, descale_q=1.0, descale_k=1.0,
                        descale_v=1.0, causal=True, out_dtype=OUT_BF16, head_dim=128, q_tile=64,
                        kv_block=64):
    return SmlaPrefillParams(batch=batch, h_q=h_q, h_kv=h_kv, head_dim=head_dim, max_s_q=max_s_q,
                             max_s_kv=max_s_kv, causal=1 if causal else 0, q_tile=q_tile, kv_block=kv_block,
                             softmax_scale=softmax_scale, descale_q=descale_q, descale_k=descale_k,
                             descale_v=descale_v, out_dtype=out_dtype)


def sdpa_fp8_prefill(q, k, v, seqlen_q, seqlen_kv, split_kv, softmax_scale, descale_q=1.0, descale_k=1.0,
                     descale_v=1.0, causal=True, sink=None, o_part=None, lse_part=None, out=None, lse_out=None,
                     amax_out=None, out_dtype=None, stream=None):
    """FP8 prefill attention through the C ABI (include/smla.h, sdpa_fp8_prefill).

    q [B, Sq, h_q, 128], k and v [B, Skv, h_kv, 128] uint8 e4m3 codes; seqlen_q / seqlen_kv [B]
    int32; the output dtype follows `out` (bf16 / float32) unless `out_dtype` is given."""
    import torch
    lib = load_library()
    B, sq_max, h_q, d = q.shape
    skv_max, h_kv = k.shape[1], k.shape[2]
    dev = q.device
    if d != 128 or tuple(k.shape) != (B, skv_max, h_kv, 128) or tuple(v.shape) != tuple(k.shape):
        raise SmlaError("q, k and v must be [B, S, heads, 128] with matching k / v")
    od = _out_dtype_of(out, out_dtype)
    codes = (torch.uint8, torch.float8_e4m3fn)
    _need(q, "q", q.numel(), codes, dev)
    _need(k, "k", k.numel(), codes, dev)
    _need(v, "v", v.numel(), codes, dev)
    _need(seqlen_q, "seqlen_q", B, (torch.int32,), dev)
    _need(seqlen_kv, "seqlen_kv", B, (torch.int32,), dev)
    _need(sink, "sink", h_q, (torch.float32,), dev)
    _need(o_part, "o_part", split_kv * B * sq_max * h_q * 128, (torch.float32,), dev)
    _need(lse_part, "lse_part", split_kv * B * sq_max * h_q, (torch.float32,), dev)
    _need(out, "out", B * sq_max * h_q * 128, {OUT_BF16: (torch.bfloat16,), OUT_FP32: (torch.float32,)}.get(
        od, (torch.bfloat16,)), dev)
    _need(lse_out, "lse_out", B * sq_max * h_q, (torch.float32,), dev)
    _need(amax_out, "amax_out", 1, (torch.float32,), dev)
    p = make_prefill_params(B, h_q, h_kv, sq_max, skv_max, softmax_scale, descale_q, descale_k, descale_v,
                            causal, od)
    st = lib.sdpa_fp8_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(seqlen_q), _ptr(seqlen_kv),
                              int(split_kv), _ptr(sink), _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse_out),
                              _ptr(amax_out), _stream_handle(stream, dev))
    _check(st, "sdpa_fp8_prefill")
