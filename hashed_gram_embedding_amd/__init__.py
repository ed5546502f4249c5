"""MI355X-native Engram conditional-memory layer (hashed n-gram embeddings).

The compute path lives in the HIP library `libengram.so` (C ABI declared in
include/engram.h); `hashed_gram_embedding_amd.engram` is its thin ctypes
binding.  `inputs` draws seeded synthetic workloads.
"""
