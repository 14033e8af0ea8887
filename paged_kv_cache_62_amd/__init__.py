"""paged_kv_cache_62_amd: paged-KV single-token decode attention for MI355X (gfx950).

The product is libpkv.so (C ABI in include/pkv.h: host block allocator plus
HIP kernels); `pkv` is its thin Python binding and `synth` the seeded
synthetic-input generator. Importing the package loads nothing; the library
is loaded on first use and raises if it has not been built.
"""
from .build import LIB, build  # noqa: F401
