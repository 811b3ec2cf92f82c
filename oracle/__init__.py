"""fp64 CPU oracle for one token-chunked DiT block (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never calls it.
"""
from .dit_block import *  # noqa: F401,F403
