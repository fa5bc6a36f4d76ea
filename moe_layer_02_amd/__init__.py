"""MI355X-native fused Mixture-of-Experts layer forward.

The compute path is the HIP library ``libmoe.so`` (built from ``csrc/``) behind the C-ABI
declared in ``include/moe.h``; ``abi`` is its thin ctypes binding.  ``synth`` draws the
seeded synthetic layers used by the tests and the benchmark.
"""
