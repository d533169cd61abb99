"""MI355X (gfx950) OneTrans hot path: HIP kernels behind a C ABI (include/onetrans.h).

The package holds the HIP sources (csrc/), their in-tree build (build.py -> libonetrans.so),
the ctypes binding (_lib.py, binding.py) and the host-side cost model (costmodel.py).
Importing the package does not load the library; the binding loads it on first use and
raises if it has not been built.
"""

__all__ = ["binding", "costmodel"]
