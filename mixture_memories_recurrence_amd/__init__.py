"""MI355X-native Mixture-of-Memories layer forward (HIP kernels behind a C ABI).

Importing the package is cheap: the HIP library is loaded on first use by
``mixture_memories_recurrence_amd.mom``.  ``synth`` holds the seeded synthetic
input generator and nothing of the layer's arithmetic.
"""
__all__ = ["synth", "mom"]
