"""MI355X (gfx950) sparse mixture-of-experts layer: HIP kernels behind a C ABI.

* ``include/moe.h``       -- the C ABI (entry points, layouts, errors)
* ``csrc/*.hip``          -- the kernels and the ABI implementation
* ``_lib``                -- ctypes binding, one function per C symbol
* ``layer.MoELayer``      -- forward/backward call sequence over torch buffers
* ``build``               -- in-tree hipcc build of ``libmoe.so``

Importing ``_lib`` (or ``layer``) requires the built library; there is no
fallback implementation.
"""
__all__ = ["build", "_lib", "layer"]
