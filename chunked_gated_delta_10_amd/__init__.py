"""KDA (Kimi Delta Attention) forward pass for AMD MI355X (gfx950).

The compute path is a set of hand-written HIP kernels behind a C ABI
(``libkda.so``, declared in ``include/kda.h``).  ``kda`` is the thin Python
binding (argument marshalling only); ``inputs`` draws seeded synthetic
workloads.  The shared library is loaded on first use, and every entry
point raises if it is missing: there is no CPU fallback.
"""

__all__ = ["kda", "inputs"]
