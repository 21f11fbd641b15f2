"""fp64 CPU oracle for factored recurrent states (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .oracle import OraclePool, build_oracle, householder_qr, jacobi_svd, brand_update, schedule_due  # noqa: F401
