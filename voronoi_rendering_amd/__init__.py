"""MI355X-native hot path of Soft Anisotropic Diagrams (SAD).

The work runs in libsad.so (HIP kernels for gfx950 behind the C ABI declared
in include/sad.h).  ``ops`` wraps each C call for torch tensors; ``pipeline``
strings the calls into a GPU-resident fitting loop.
"""
from . import _native, ops  # noqa: F401

__all__ = ["ops", "pipeline"]
