"""librocs: MI355X (gfx950) implementation of the ROCS shared forward pass.

``rocs``    ctypes binding of the C ABI declared in include/rocs.h
``stacks``  device-side descriptors of the five benchmark workloads
``build``   in-tree hipcc build of librocs.so

The computation lives entirely in librocs's HIP kernels; importing this
package does not load the library, the first call does (and raises if the
library has not been built).
"""

from . import rocs  # noqa: F401

__all__ = ["rocs"]
