"""MI355X-native QEvict decode hot path: HIP kernels behind a C ABI, with a thin ctypes binding.

Importing the package loads nothing; ``recoverable_kv_cache_amd.binding`` loads the HIP library.
"""
