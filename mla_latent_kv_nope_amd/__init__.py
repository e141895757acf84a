"""MI355X-native MLA absorbed decode over a paged latent cache.

The compute lives in libmla.so (HIP kernels for gfx950 behind the C ABI of
include/mla.h); this package is its Python binding.  Importing it loads the
library and fails if it is missing.
"""
from ._native import LIB_PATH, Dims  # noqa: F401
from .api import (  # noqa: F401
    MlaError, absorb_q, append_latent, cache_bytes_per_token, decode_paged, decode_workspace_size,
    make_dims, new_pool, new_workspace, out_proj, pool_shape, profile_begin, profile_end,
    status_string,
)
