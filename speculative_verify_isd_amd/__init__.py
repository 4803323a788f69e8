"""MI355X-native ISD verify-and-propose step.

``libidlm_isd.so`` (built from ``csrc/``) holds the HIP kernels and the C ABI
declared in ``include/idlm_isd.h``.  ``speculative_verify_isd_amd.lib`` is a
thin ctypes binding with the same entry-point names; ``workloads`` draws
seeded synthetic inputs.  The binding is imported lazily so that input
generation works on machines without the library.
"""

__all__ = ["lib", "workloads", "build"]
