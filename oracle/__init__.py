"""Float64 CPU oracles (test infrastructure only): split-KV sparse MLA decode
(``smla_oracle``, re-exported here) and split-KV FP8 prefill attention
(``oracle.prefill_oracle``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .smla_oracle import *  # noqa: F401,F403
from .smla_oracle import __doc__ as _doc  # noqa: F401
