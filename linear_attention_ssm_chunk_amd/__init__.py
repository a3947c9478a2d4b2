"""MI355X-native chunked gated-delta-rule (Gated DeltaNet) prefill.

The compute path is ``libgdn_prefill.so``: three HIP kernels for gfx950 behind
a C ABI (``include/gdn_prefill.h``).  ``binding`` wraps that ABI with ctypes
(argument marshalling only); ``inputs`` draws seeded synthetic problems.
"""
