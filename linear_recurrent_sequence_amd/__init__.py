"""Multi-scale retention (RetNet) for MI355X: HIP kernels behind a C ABI, with a thin Python binding.

The binding (``linear_recurrent_sequence_amd.retention``) is imported on demand so that the seeded input
module can be used without torch or the built library.
"""

__all__ = ["workloads", "retention"]
