"""W12 oracle package: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. It never imports the HIP library or its binding,
and the library never calls it.
"""
from .w12_ref import *  # noqa: F401,F403
from .w12_ref import Encoded, ESC_DTYPE  # noqa: F401
