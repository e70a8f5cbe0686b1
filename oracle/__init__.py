"""Plain CPU oracle for the MoE-layer hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` are the only users.  Nothing here is imported by
the HIP path, and this package imports nothing from it.

Parity status per function is listed in the header of ``oracle.py``.
"""
from .oracle import *  # noqa: F401,F403
