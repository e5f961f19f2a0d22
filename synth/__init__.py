"""Seeded synthetic inputs for the CSA/HCA attention core.

This package is shared by the oracle-based tests, ``bench.py`` and
``__graft_entry__.smoke()``.  It draws random numbers and stores them in the
dtypes the path reads (fp32, bf16, OCP e4m3fn plus a per-row fp32 scale).  It
holds none of the method's arithmetic: no pooling, no scores, no selection, no
attention, no normalisation and no rotation.
"""
from .gen import Gen, quantize_rows_e4m3, SEED_BASE  # noqa: F401
from .workloads import WORKLOADS, Workload  # noqa: F401
