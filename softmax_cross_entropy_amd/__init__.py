"""MI355X-native fused softmax cross-entropy.

The compute lives in ``libce_mi355x.so`` (hand-written HIP for gfx950 behind a
C ABI declared in ``include/ce_mi355x.h``).  ``softmax_cross_entropy_amd.abi``
is the thin ctypes binding with the same entry-point names; importing this
package does not load the library, so the input generators in ``inputs`` work
on machines without a GPU.
"""

__all__ = ["abi", "inputs"]
