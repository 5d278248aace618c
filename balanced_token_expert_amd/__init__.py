"""MI355X-native forward pass of a BASE (balanced assignment of experts) layer.

The compute path is a C-ABI shared library of hand-written gfx950 HIP kernels
(``libbase_layer.so``, declared in ``include/base_layer.h``). This package's
``api`` module is a thin ctypes binding over it: argument marshalling only,
with torch used for device memory and streams. The library is loaded on the
first call; if it is missing the call raises, there is no fallback.
"""

__all__ = ["api", "workloads"]
