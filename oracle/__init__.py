"""Float64 CPU oracle for split-KV sparse MLA decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .smla_oracle import *  # noqa: F401,F403
from .smla_oracle import __doc__ as _doc  # noqa: F401
