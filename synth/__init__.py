"""Seeded synthetic workloads shared by the GPU tests, the benchmark and the oracle tests.

Holds no attention arithmetic: random draws, storage rounding and paged layout only.
"""

from .configs import DECODE_WORKLOADS, PREFILL_WORKLOADS, WORKLOADS  # noqa: F401
from .workloads import alibi_slopes_pow2, make_case  # noqa: F401
