"""paged_kv_cache_356_amd — decode-step paged attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libpa.so`` (hand-written HIP kernels behind the C ABI in
``include/pa.h``); ``api`` is a thin ctypes binding with the same names.  Importing the package does
not load the library: the first call into ``api`` does, and raises if it is not built.
"""

__all__ = ["api", "workloads"]
