"""MI355X-native group-wise affine quantized linear (y = x @ W_hat^T).

The compute path is the HIP/C library ``libqlinear.so`` (built from ``csrc/``);
``qlinear`` is a thin ctypes binding over its C ABI. Importing this package
does not load the library; the first call does, and fails loudly if it is not
built.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs"]
