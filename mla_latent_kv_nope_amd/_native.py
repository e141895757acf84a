"""Loads libmla.so (built in-tree by mla_latent_kv_nope_amd.build) and declares
the C ABI of include/mla.h for ctypes.  There is no fallback: if the library
is missing or does not load, importing the package fails with the reason."""
from __future__ import annotations

import ctypes
import os

# PyTorch wheels bundle their own HIP runtime.  Importing torch first puts that
# runtime in the process, so libmla's libamdhip64.so.7 dependency resolves to
# the same copy; loading libmla first would bring in a second HIP runtime that
# cannot use torch's device pointers and streams.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB_PATH selects another build of the same library (the sanitized build
# of the host-only ABI tests); by default the in-tree libmla.so
LIB_PATH = os.environ.get("MLA_LIB_PATH") or os.path.join(_HERE, "libmla.so")


class Dims(ctypes.Structure):
    """mla_dims_t (40 bytes)."""
    _fields_ = [
        ("n_heads", ctypes.c_int32),
        ("d_c", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_double),
    ]


assert ctypes.sizeof(Dims) == 40

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
MLA_CACHE_BF16 = 0
MLA_CACHE_FP8_E4M3 = 1
MLA_APPEND_NO_ROPE = 1
MLA_MAX_Q_LEN = 16

EXPORTS = (
    "mla_append_latent", "mla_absorb_q", "mla_decode_workspace_size", "mla_decode_paged",
    "mla_decode_paged_multi", "mla_project_append", "mla_project_append_workspace_size",
    "mla_out_proj", "mla_cache_bytes_per_token", "mla_status_string", "mla_last_hip_error",
    "mla_decode_paged_timed", "mla_prefill_paged_timed", "mla_decode_paged_noalloc",
    "mla_decode_noalloc_max_bytes", "mla_prefill_workspace_size", "mla_prefill_paged",
    "mla_decode_paged_out", "mla_append_absorb",
)

_P = ctypes.c_void_p
_I = ctypes.c_int32
_DP = ctypes.POINTER(Dims)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_nope_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP implementation")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_append_latent.argtypes = [_DP, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P,
                                      ctypes.c_uint32, _P]
    lib.mla_append_latent.restype = ctypes.c_int
    lib.mla_absorb_q.argtypes = [_DP, _P, _P, _P, _P, _I, _P, _P]
    lib.mla_absorb_q.restype = ctypes.c_int
    lib.mla_append_absorb.argtypes = [_DP, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, ctypes.c_uint32,
                                      _P, _P, _P, _P, _I, _P, _P]
    lib.mla_append_absorb.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [_DP, _I, _I]
    lib.mla_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode_paged.argtypes = [_DP, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P, ctypes.c_size_t,
                                     _P, _P, _P]
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_decode_paged_multi.argtypes = [_DP, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P,
                                           ctypes.c_size_t, _P, _P, _P]
    lib.mla_decode_paged_multi.restype = ctypes.c_int
    lib.mla_project_append_workspace_size.argtypes = [_DP, _I, _I]
    lib.mla_project_append_workspace_size.restype = ctypes.c_size_t
    lib.mla_project_append.argtypes = [_DP, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P,
                                       ctypes.c_size_t, _P]
    lib.mla_project_append.restype = ctypes.c_int
    lib.mla_prefill_workspace_size.argtypes = [_DP, _I, _I]
    lib.mla_prefill_workspace_size.restype = ctypes.c_size_t
    lib.mla_prefill_paged.argtypes = [_DP, _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P, _P,
                                      _P, ctypes.c_size_t, _P, _P, _P]
    lib.mla_prefill_paged.restype = ctypes.c_int
    lib.mla_out_proj.argtypes = [_DP, _P, _P, _I, _P, _P]
    lib.mla_out_proj.restype = ctypes.c_int
    lib.mla_cache_bytes_per_token.argtypes = [_DP]
    lib.mla_cache_bytes_per_token.restype = ctypes.c_size_t
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_hip_error.argtypes = []
    lib.mla_last_hip_error.restype = ctypes.c_char_p
    lib.mla_decode_paged_timed.argtypes = [_DP, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P,
                                           ctypes.c_size_t, _P, _P, _P, _P, _P]
    lib.mla_decode_paged_timed.restype = ctypes.c_int
    lib.mla_decode_paged_out.argtypes = [_DP, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P,
                                         ctypes.c_size_t, _P, _P, _P, _P, _P, _P]
    lib.mla_decode_paged_out.restype = ctypes.c_int
    lib.mla_decode_paged_noalloc.argtypes = [_DP, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P]
    lib.mla_decode_paged_noalloc.restype = ctypes.c_int
    lib.mla_decode_noalloc_max_bytes.argtypes = []
    lib.mla_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.mla_prefill_paged_timed.argtypes = [_DP, _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P, _P,
                                            _P, ctypes.c_size_t, _P, _P, _P, _P, _P]
    lib.mla_prefill_paged_timed.restype = ctypes.c_int
    return lib


lib = _load()
