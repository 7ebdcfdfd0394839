"""aqkv: compressed KV-cache key quantisation and decode attention on packed
bits, for AMD Instinct MI355X (gfx950).

The compute path is ``libaqkv.so`` (hand-written HIP kernels behind a C ABI,
``include/aqkv.h``); ``kv_cache_compression_quantize_amd.aqkv`` is its thin
ctypes binding.  Importing this package loads nothing; the library is loaded
on first use and a missing build is an error, never a fallback.
"""
