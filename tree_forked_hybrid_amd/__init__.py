"""MI355X-native ForkAttention hot path: HIP kernels for gfx950 behind a C ABI (libflide.so).

``flide``  — ctypes binding with the C entry points' names (marshalling only)
``runner`` — torch-allocated device buffers of a round (imports torch)
``build``  — in-tree hipcc build of libflide.so

There is no CPU fallback: every call goes to libflide.so, and loading fails
with an ImportError when the library has not been built.
"""
from . import flide  # noqa: F401
from .flide import FlideError, load_library  # noqa: F401
