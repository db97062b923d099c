"""Paged-attention read path for AMD MI355X (gfx950): HIP kernels behind the
C ABI of include/pa.h, with a thin torch binding.

``import paged_kv_cache_96_amd`` itself needs neither torch nor a GPU; the
binding (``paged_kv_cache_96_amd.api``) loads libpa.so and fails loudly if
it has not been built.
"""
from ._lib import LIB_PATH, EXPORTED  # noqa: F401

__all__ = ["LIB_PATH", "EXPORTED"]
