"""fp64 CPU oracle — test infrastructure only (see ``oracle/ref.py``).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg import this package.  The HIP library never does.
"""
from .ref import (combine, diag_scan, diag_scan_bwd, discretize, discretize_grads,  # noqa: F401
                  selective_scan, selective_scan_bwd, ssd_scan, ssd_scan_bwd, gla_scan, gla_scan_bwd, rotlru_scan,
                  rotlru_scan_bwd)
from .metrics import max_rel_err, rel_err_p99, rel_err_p999, rel_err_pct  # noqa: F401
