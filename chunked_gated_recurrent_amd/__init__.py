"""Simple GLA (fixed per-head decay, matrix state) for AMD MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libgla.so``, declared in ``include/gla.h``); ``gla`` is its thin Python
binding and ``workloads`` the seeded synthetic inputs. Importing the package
loads nothing; the library is loaded on first use of the binding.
"""
__all__ = ["gla", "workloads"]
