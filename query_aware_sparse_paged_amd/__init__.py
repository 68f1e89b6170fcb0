"""query_aware_sparse_paged_amd: one decode step of query-aware sparse
attention over a paged KV cache, as hand-written HIP kernels for gfx950 behind
a C ABI (``include/qasp.h``), with a thin ctypes binding.

The binding (``query_aware_sparse_paged_amd.api``) loads ``libqasp.so`` on
first use and raises if it is missing: there is no CPU fallback.
"""

__all__ = ["api", "workloads"]
