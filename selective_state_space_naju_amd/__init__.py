"""MI355X-native Naju selective state scan.

The compute path is the HIP library ``libnaju.so`` (hand-written gfx950
kernels behind the C ABI declared in ``include/naju.h``).  The Python side is
argument marshalling only: see ``binding.py``.  ``inputs.py`` draws seeded
synthetic workloads and holds none of the method's arithmetic.
"""
__all__ = ["binding", "inputs"]
