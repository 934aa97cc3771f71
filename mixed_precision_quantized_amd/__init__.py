"""MI355X-native mixed-precision quantized KV cache.

Low-bit block formats (qN_0, qN_1, kvarnN) with a BF16 precision tail, appended and
read by hand-written HIP kernels for gfx950 behind a small C ABI (libkvq.so).  The
Python side only marshals arguments: see `mixed_precision_quantized_amd.kvq`.

Importing this package loads nothing; `kvq` loads the HIP library on first use and
raises if it is missing (there is no CPU fallback).
"""
__all__ = ["kvq", "synth"]
