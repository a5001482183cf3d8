"""ZHA decode path on MI355X: summary-tree build/append, top-down top-p routing,
sparse exact attention and a dense decode baseline, as HIP kernels for gfx950
behind the C ABI of include/zha.h (libzha.so).  `zha` is the ctypes binding;
`runtime` holds torch-side helpers that allocate buffers and call it.
"""
from . import zha  # noqa: F401
