"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package draws random numbers, rounds them to the storage precision and
(for the clustered workload) orders tokens by cluster label. It holds none of
the attention arithmetic: both sides receive the same arrays and compute on
their own.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from . import gen  # noqa: F401
