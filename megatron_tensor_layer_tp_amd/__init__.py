"""MI355X-native shard of a Megatron-style tensor-parallel transformer layer.

The compute lives in libtpshard.so (hand-written HIP for gfx950, C ABI in
include/tpshard.h); ``tpshard`` is its thin ctypes binding, ``inputs`` the
seeded synthetic input generator.  Importing the package loads nothing.
"""
__all__ = ["tpshard", "inputs", "build"]
