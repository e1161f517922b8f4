"""Packed 2-bit ternary KV cache with direct decode attention, for MI355X (gfx950).

The compute lives in libvk.so (hand-written HIP kernels behind a C ABI);
this package only marshals arguments (``vk``), builds the library (``build``)
and draws seeded synthetic workloads (``workloads``).
"""
from .vk import (Cache, CacheConfig, VkError, make_config, device_bytes, page_bytes,  # noqa: F401
                 quantize_pack, DTYPE_F16, DTYPE_BF16, FMT_TERNARY2, FMT_FP8E4M3, FMT_F16)
