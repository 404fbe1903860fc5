"""CPU oracle for quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library and imports nothing from it.

Every function is pinned by ``tests/test_oracle_*.py`` against facts the pages
and the mathematics fix (closed forms, invariants, special cases that reduce to
library routines, brute force on tiny inputs).  Parity status per function is
listed in the module docstring of :mod:`oracle.kvq_oracle`.
"""
from .kvq_oracle import *  # noqa: F401,F403
