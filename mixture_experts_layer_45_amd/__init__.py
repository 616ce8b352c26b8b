"""MI355X-native forward pass of one sparse mixture-of-experts layer.

The layer runs as hand-written HIP kernels for gfx950 behind a C ABI
(include/moe.h, built into libmoe.so).  This package is the thin Python
binding over that ABI (argument marshalling only) plus the seeded input
generators; PyTorch supplies device memory and streams.
"""
