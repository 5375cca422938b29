"""pagedkv on MI355X: paged KV cache and decode attention (gfx950 HIP kernels, C ABI).

The compute runs in libpagedkv.so (include/pagedkv.h); this package only loads
it and marshals arguments. Build it first: python -m paged_kv_cache_320_amd.build
"""
from . import _lib
from ._lib import (PA_BF16, PA_EHIP, PA_EINVAL, PA_ENOBLOCKS, PA_ENOSEQ, PA_EUNSUPPORTED, PA_F16,
                   PA_F32, PA_OK, PagedKVError)
from .cache import BlockAllocator, PagedKVCache, torch_dtype

__all__ = ["_lib", "BlockAllocator", "PagedKVCache", "PagedKVError", "torch_dtype", "PA_OK",
           "PA_EINVAL", "PA_ENOBLOCKS", "PA_ENOSEQ", "PA_EHIP", "PA_EUNSUPPORTED", "PA_F32",
           "PA_F16", "PA_BF16"]
