"""MI355X-native MLA absorbed decode over a paged latent cache.

The compute lives in libmla.so (HIP kernels for gfx950 behind the C ABI of
include/mla.h); this package is its Python binding.  The library is loaded on
first use of any binding attribute, and that use fails (ImportError) if the
library is missing; `mla_latent_kv_nope_amd.build` builds it.
"""
_API = (
    "Dims", "LIB_PATH", "MlaError", "absorb_q", "append_absorb", "append_latent", "cache_bytes_per_token",
    "decode_paged", "decode_paged_multi", "decode_paged_noalloc", "decode_noalloc_max_bytes",
    "decode_paged_out",
    "decode_workspace_size", "make_dims", "new_pool",
    "new_workspace", "out_proj", "prefill_paged", "prefill_workspace_size", "project_append",
    "project_append_workspace_size",
    "pool_shape", "status_string",
)
__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import api, _native
        return getattr(api, name) if hasattr(api, name) else getattr(_native, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
