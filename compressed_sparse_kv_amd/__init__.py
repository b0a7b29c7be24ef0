"""CSA / HCA attention hot path (DeepSeek-V4 compressed sparse attention) for MI355X.

The compute lives in the HIP library ``libcsa.so`` (C ABI: ``include/csa.h``);
``compressed_sparse_kv_amd.binding`` exposes its entry points to Python with the
same names.  Build with ``python -m compressed_sparse_kv_amd.build``.
"""

__all__ = ["binding", "build"]
