"""Split-KV sparse MLA decode for MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C-ABI shared library
(``include/smla.h``); this package is the thin ctypes binding to it plus the
seeded input generators.  The library is loaded on first use and its absence
is an error: there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    SmlaError, KV_BF16, KV_FP8_E4M3, OUT_BF16, OUT_FP32, OUT_FP8_E4M3,
    library_path, load_library, sparse_mla_decode, sparse_mla_decode_noalloc, combine_splits,
    smla_choose_num_splits, smla_partial_bytes, smla_validate, smla_status_string,
    sdpa_fp8_prefill, smla_prefill_partial_bytes, smla_prefill_choose_splits,
)
