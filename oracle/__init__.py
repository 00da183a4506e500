"""Plain, slow fp64 CPU oracle for the BCQ LUT-GEMV.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path: the only thing both sides use is the seeded input generator in
``workloads``.

Parity status per function is listed in the module docstring of
``oracle.bcq``.
"""
from .bcq import *  # noqa: F401,F403
from .bcq import __all__  # noqa: F401
