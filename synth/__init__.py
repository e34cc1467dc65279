"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This package holds random draws, their encoding into the storage formats (torch casts) and their
placement into pages. It holds none of the DSA arithmetic: no scores, no selection, no attention.
"""
from .workloads import (  # noqa: F401
    Workload,
    make_workload,
    WORKLOADS,
    index_page_bytes,
    latent_row_bytes,
)
from .msa_workloads import MsaWorkload, make_msa_workload, MSA_WORKLOADS  # noqa: F401,E402
