"""CPU oracle for LB-ADMM (test infrastructure only; see oracle.lbadmm).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` import this package. The GPU library never does.
"""
from . import binary, brute, lbadmm, precond, ste  # noqa: F401
