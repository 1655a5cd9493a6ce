"""MI355X-native streaming-prefill attention over a view-major, pre-RoPE KV cache.

The compute path is the HIP library `libfdattn.so` (C ABI declared in
`include/fdattn.h`); `streaming_kv_cache_view_amd.fd` is its thin ctypes
binding.  `streaming_kv_cache_view_amd.synth` holds the seeded synthetic
inputs.  Importing this package loads neither.
"""
__all__ = ["fd", "synth"]
