"""Python binding of libmla: argument marshalling only.

Each function checks tensor dtypes, shapes, devices and contiguity, then calls
the C entry point of the same name with raw device pointers and torch's
current HIP stream.  Every step of MLA decode runs in the library's kernels;
PyTorch only provides device memory and the stream.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _native
from ._native import Dims, lib


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = f"{fn} failed: {status_string(status)}"
        if status == _native.MLA_ERR_HIP:
            msg += f" ({lib.mla_last_hip_error().decode()})"
        super().__init__(msg)


def status_string(status: int) -> str:
    return lib.mla_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != _native.MLA_OK:
        raise MlaError(fn, status)


def make_dims(n_heads: int, d_c: int, d_rope: int, d_nope: int, d_v: int, page_size: int,
              fp8: bool = False, softmax_scale: Optional[float] = None,
              rope_base: float = 10000.0) -> Dims:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_nope + d_rope)
    return Dims(n_heads, d_c, d_rope, d_nope, d_v, page_size,
                _native.MLA_CACHE_FP8_E4M3 if fp8 else _native.MLA_CACHE_BF16,
                float(softmax_scale), float(rope_base))


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _event_handles(events) -> Tuple[Optional[int], Optional[int]]:
    """(start, stop) torch.cuda.Event pair -> raw hipEvent_t handles.  A torch
    event creates its HIP event at its first record, so an uncreated one is
    recorded once here first; the library then records it again on the call's
    stream around the main kernel."""
    if events is None:
        return None, None
    out = []
    for ev in events:
        if not isinstance(ev, torch.cuda.Event):
            raise TypeError("events must be a pair of torch.cuda.Event")
        if not ev.cuda_event:
            ev.record()
        out.append(ev.cuda_event)
    return out[0], out[1]


def _req(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Optional[tuple] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _is_fp8(d: Dims) -> bool:
    return d.cache_dtype == _native.MLA_CACHE_FP8_E4M3


def pool_shape(d: Dims, num_pages: int) -> tuple:
    return (num_pages, d.page_size, d.d_c + d.d_rope)


def new_pool(d: Dims, num_pages: int, device="cuda") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Allocate an (uninitialised) cache pool and, for fp8, its scale array."""
    if _is_fp8(d):
        return (torch.empty(pool_shape(d, num_pages), dtype=torch.uint8, device=device),
                torch.empty((num_pages, d.page_size), dtype=torch.float32, device=device))
    return torch.empty(pool_shape(d, num_pages), dtype=torch.bfloat16, device=device), None


def append_latent(d: Dims, c_kv: torch.Tensor, k_pe: torch.Tensor, positions: torch.Tensor,
                  seq_ids: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                  scales: Optional[torch.Tensor] = None, rope: bool = True) -> None:
    T = c_kv.shape[0]
    _req(c_kv, "c_kv", torch.bfloat16, (T, d.d_c))
    _req(k_pe, "k_pe", torch.bfloat16, (T, d.d_rope))
    _req(positions, "positions", torch.int32, (T,))
    _req(seq_ids, "seq_ids", torch.int32, (T,))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs][max_pages]")
    _req(block_table, "block_table", torch.int32)
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        if scales is None:
            raise ValueError("an fp8 cache needs its scales tensor")
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
        if scales is not None:
            raise ValueError("a bf16 cache has no scales")
    st = lib.mla_append_latent(
        ctypes.byref(d), _ptr(c_kv), _ptr(k_pe), _ptr(positions), _ptr(seq_ids), _ptr(block_table),
        block_table.shape[0], block_table.shape[1], num_pages, T, _ptr(pool), _ptr(scales),
        0 if rope else _native.MLA_APPEND_NO_ROPE, _stream())
    _check("mla_append_latent", st)


def project_append_workspace_size(d: Dims, d_model: int, n_tokens: int) -> int:
    return int(lib.mla_project_append_workspace_size(ctypes.byref(d), int(d_model), int(n_tokens)))


def project_append(d: Dims, h: torch.Tensor, w_down: torch.Tensor, positions: torch.Tensor,
                   seq_ids: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                   scales: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> None:
    """mla_project_append: h [T][d_model], w_down [d_c + d_rope][d_model] (bf16)."""
    T, d_model = h.shape[0], h.shape[1]
    R = d.d_c + d.d_rope
    _req(h, "h", torch.bfloat16, (T, d_model))
    _req(w_down, "w_down", torch.bfloat16, (R, d_model))
    _req(positions, "positions", torch.int32, (T,))
    _req(seq_ids, "seq_ids", torch.int32, (T,))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs][max_pages]")
    _req(block_table, "block_table", torch.int32)
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        if scales is None:
            raise ValueError("an fp8 cache needs its scales tensor")
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if workspace is None:
        n = project_append_workspace_size(d, d_model, T)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=h.device)
    _req(workspace, "workspace", torch.uint8)
    st = lib.mla_project_append(ctypes.byref(d), d_model, _ptr(h), _ptr(w_down), _ptr(positions),
                                _ptr(seq_ids), _ptr(block_table), block_table.shape[0],
                                block_table.shape[1], num_pages, T, _ptr(pool), _ptr(scales),
                                _ptr(workspace), workspace.numel(), _stream())
    _check("mla_project_append", st)


def absorb_q(d: Dims, q_nope: torch.Tensor, q_pe: torch.Tensor, q_pos: torch.Tensor,
             w_uk: torch.Tensor, q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    B = q_nope.shape[0]
    H = d.n_heads
    _req(q_nope, "q_nope", torch.bfloat16, (B, H, d.d_nope))
    _req(q_pe, "q_pe", torch.bfloat16, (B, H, d.d_rope))
    _req(q_pos, "q_pos", torch.int32, (B,))
    _req(w_uk, "w_uk", torch.bfloat16, (H, d.d_c, d.d_nope))
    if q_out is None:
        q_out = torch.empty((B, H, d.d_c + d.d_rope), dtype=torch.bfloat16, device=q_nope.device)
    _req(q_out, "q_out", torch.bfloat16, (B, H, d.d_c + d.d_rope))
    _check("mla_absorb_q", lib.mla_absorb_q(ctypes.byref(d), _ptr(q_nope), _ptr(q_pe), _ptr(q_pos),
                                            _ptr(w_uk), B, _ptr(q_out), _stream()))
    return q_out


def append_absorb(d: Dims, c_kv: torch.Tensor, k_pe: torch.Tensor, positions: torch.Tensor,
                  seq_ids: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                  scales: Optional[torch.Tensor], q_nope: torch.Tensor, q_pe: torch.Tensor,
                  q_pos: torch.Tensor, w_uk: torch.Tensor, q_out: Optional[torch.Tensor] = None,
                  rope: bool = True) -> torch.Tensor:
    """mla_append_absorb: append_latent(c_kv, k_pe, ...) and absorb_q(q_nope,
    q_pe, q_pos, w_uk) in one launch; returns q_out."""
    T = c_kv.shape[0]
    _req(c_kv, "c_kv", torch.bfloat16, (T, d.d_c))
    _req(k_pe, "k_pe", torch.bfloat16, (T, d.d_rope))
    _req(positions, "positions", torch.int32, (T,))
    _req(seq_ids, "seq_ids", torch.int32, (T,))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs][max_pages]")
    _req(block_table, "block_table", torch.int32)
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        if scales is None:
            raise ValueError("an fp8 cache needs its scales tensor")
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
        if scales is not None:
            raise ValueError("a bf16 cache has no scales")
    B = q_nope.shape[0]
    H = d.n_heads
    _req(q_nope, "q_nope", torch.bfloat16, (B, H, d.d_nope))
    _req(q_pe, "q_pe", torch.bfloat16, (B, H, d.d_rope))
    _req(q_pos, "q_pos", torch.int32, (B,))
    _req(w_uk, "w_uk", torch.bfloat16, (H, d.d_c, d.d_nope))
    if q_out is None:
        q_out = torch.empty((B, H, d.d_c + d.d_rope), dtype=torch.bfloat16, device=q_nope.device)
    _req(q_out, "q_out", torch.bfloat16, (B, H, d.d_c + d.d_rope))
    st = lib.mla_append_absorb(
        ctypes.byref(d), _ptr(c_kv), _ptr(k_pe), _ptr(positions), _ptr(seq_ids), _ptr(block_table),
        block_table.shape[0], block_table.shape[1], num_pages, T, _ptr(pool), _ptr(scales),
        0 if rope else _native.MLA_APPEND_NO_ROPE, _ptr(q_nope), _ptr(q_pe), _ptr(q_pos), _ptr(w_uk), B,
        _ptr(q_out), _stream())
    _check("mla_append_absorb", st)
    return q_out


def decode_workspace_size(d: Dims, B: int, num_splits: int = 0) -> int:
    n = lib.mla_decode_workspace_size(ctypes.byref(d), int(B), int(num_splits))
    if n == 0:
        raise MlaError("mla_decode_workspace_size", _native.MLA_ERR_UNSUPPORTED)
    return int(n)


def new_workspace(d: Dims, B: int, num_splits: int = 0, device="cuda") -> torch.Tensor:
    return torch.empty(decode_workspace_size(d, B, num_splits), dtype=torch.uint8, device=device)


def decode_paged(d: Dims, q: torch.Tensor, pool: torch.Tensor, scales: Optional[torch.Tensor],
                 block_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, want_lse: bool = True, events=None):
    """mla_decode_paged; with `events` = (start, stop) torch.cuda.Event, the call
    goes through mla_decode_paged_timed and the events bracket the split kernel."""
    B = q.shape[0]
    H, R = d.n_heads, d.d_c + d.d_rope
    _req(q, "q", torch.bfloat16, (B, H, R))
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    _req(block_table, "block_table", torch.int32)
    _req(seq_lens, "seq_lens", torch.int32, (B,))
    if workspace is None:
        workspace = new_workspace(d, B, num_splits, q.device)
    _req(workspace, "workspace", torch.uint8)
    if o_lat is None:
        o_lat = torch.empty((B, H, d.d_c), dtype=torch.bfloat16, device=q.device)
    _req(o_lat, "o_lat", torch.bfloat16, (B, H, d.d_c))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _req(lse, "lse", torch.float32, (B, H))
    if events is None:
        st = lib.mla_decode_paged(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales), _ptr(block_table),
                                  block_table.shape[1], num_pages, _ptr(seq_lens), B, int(num_splits),
                                  _ptr(workspace), workspace.numel(), _ptr(o_lat), _ptr(lse), _stream())
        _check("mla_decode_paged", st)
    else:
        e0, e1 = _event_handles(events)
        st = lib.mla_decode_paged_timed(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales),
                                        _ptr(block_table), block_table.shape[1], num_pages,
                                        _ptr(seq_lens), B, 1, int(num_splits), _ptr(workspace),
                                        workspace.numel(), _ptr(o_lat), _ptr(lse), e0, e1, _stream())
        _check("mla_decode_paged_timed", st)
    return o_lat, lse


def decode_paged_multi(d: Dims, q: torch.Tensor, pool: torch.Tensor, scales: Optional[torch.Tensor],
                       block_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int = 0,
                       workspace: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, want_lse: bool = True, events=None):
    """mla_decode_paged_multi: q is [B][q_len][H][R]; returns o_lat [B][q_len][H][d_c]
    and lse [B][q_len][H] (or None)."""
    if q.dim() != 4:
        raise ValueError("q must be [B][q_len][H][d_c + d_rope]")
    B, q_len = q.shape[0], q.shape[1]
    H, R = d.n_heads, d.d_c + d.d_rope
    _req(q, "q", torch.bfloat16, (B, q_len, H, R))
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    _req(block_table, "block_table", torch.int32)
    _req(seq_lens, "seq_lens", torch.int32, (B,))
    if workspace is None:
        workspace = new_workspace(d, B * q_len, num_splits, q.device)
    _req(workspace, "workspace", torch.uint8)
    if o_lat is None:
        o_lat = torch.empty((B, q_len, H, d.d_c), dtype=torch.bfloat16, device=q.device)
    _req(o_lat, "o_lat", torch.bfloat16, (B, q_len, H, d.d_c))
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _req(lse, "lse", torch.float32, (B, q_len, H))
    if events is None:
        st = lib.mla_decode_paged_multi(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales),
                                        _ptr(block_table), block_table.shape[1], num_pages,
                                        _ptr(seq_lens), B, int(q_len), int(num_splits), _ptr(workspace),
                                        workspace.numel(), _ptr(o_lat), _ptr(lse), _stream())
        _check("mla_decode_paged_multi", st)
    else:
        e0, e1 = _event_handles(events)
        st = lib.mla_decode_paged_timed(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales),
                                        _ptr(block_table), block_table.shape[1], num_pages,
                                        _ptr(seq_lens), B, int(q_len), int(num_splits), _ptr(workspace),
                                        workspace.numel(), _ptr(o_lat), _ptr(lse), e0, e1, _stream())
        _check("mla_decode_paged_timed", st)
    return o_lat, lse


def decode_paged_noalloc(d: Dims, q: torch.Tensor, pool: torch.Tensor, scales: Optional[torch.Tensor],
                         block_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int = 0,
                         o_lat: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         want_lse: bool = True):
    """mla_decode_paged_noalloc: q is [B][H][R] (one new token per sequence) or
    [B][q_len][H][R]; the workspace is the library's device scratch array.
    Returns o_lat and lse shaped like q's leading dimensions."""
    H, R = d.n_heads, d.d_c + d.d_rope
    if q.dim() == 3:
        B, q_len = q.shape[0], 1
        lead = (B,)
    elif q.dim() == 4:
        B, q_len = q.shape[0], q.shape[1]
        lead = (B, q_len)
    else:
        raise ValueError("q must be [B][H][R] or [B][q_len][H][R]")
    _req(q, "q", torch.bfloat16, lead + (H, R))
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    _req(block_table, "block_table", torch.int32)
    _req(seq_lens, "seq_lens", torch.int32, (B,))
    if o_lat is None:
        o_lat = torch.empty(lead + (H, d.d_c), dtype=torch.bfloat16, device=q.device)
    _req(o_lat, "o_lat", torch.bfloat16, lead + (H, d.d_c))
    if lse is None and want_lse:
        lse = torch.empty(lead + (H,), dtype=torch.float32, device=q.device)
    if lse is not None:
        _req(lse, "lse", torch.float32, lead + (H,))
    st = lib.mla_decode_paged_noalloc(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales),
                                      _ptr(block_table), block_table.shape[1], num_pages, _ptr(seq_lens),
                                      B, int(q_len), int(num_splits), _ptr(o_lat), _ptr(lse), _stream())
    _check("mla_decode_paged_noalloc", st)
    return o_lat, lse


def decode_paged_out(d: Dims, q: torch.Tensor, pool: torch.Tensor, scales: Optional[torch.Tensor],
                     block_table: torch.Tensor, seq_lens: torch.Tensor, w_uv: torch.Tensor,
                     num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_o_lat: bool = False, want_lse: bool = False,
                     events=None):
    """mla_decode_paged_out: decode plus the W_UV projection in one call.  q is
    [B][H][R] or [B][q_len][H][R]; returns out [.., H, d_v], o_lat [.., H, d_c]
    (or None) and lse [.., H] (or None), shaped like q's leading dimensions."""
    H, R = d.n_heads, d.d_c + d.d_rope
    if q.dim() == 3:
        B, q_len = q.shape[0], 1
        lead = (B,)
    elif q.dim() == 4:
        B, q_len = q.shape[0], q.shape[1]
        lead = (B, q_len)
    else:
        raise ValueError("q must be [B][H][R] or [B][q_len][H][R]")
    _req(q, "q", torch.bfloat16, lead + (H, R))
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    _req(block_table, "block_table", torch.int32)
    _req(seq_lens, "seq_lens", torch.int32, (B,))
    _req(w_uv, "w_uv", torch.bfloat16, (H, d.d_c, d.d_v))
    if workspace is None:
        workspace = new_workspace(d, B * q_len, num_splits, q.device)
    _req(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty(lead + (H, d.d_v), dtype=torch.bfloat16, device=q.device)
    _req(out, "out", torch.bfloat16, lead + (H, d.d_v))
    if o_lat is None and want_o_lat:
        o_lat = torch.empty(lead + (H, d.d_c), dtype=torch.bfloat16, device=q.device)
    if o_lat is not None:
        _req(o_lat, "o_lat", torch.bfloat16, lead + (H, d.d_c))
    if lse is None and want_lse:
        lse = torch.empty(lead + (H,), dtype=torch.float32, device=q.device)
    if lse is not None:
        _req(lse, "lse", torch.float32, lead + (H,))
    e0, e1 = _event_handles(events) if events is not None else (None, None)
    st = lib.mla_decode_paged_out(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(scales), _ptr(block_table),
                                  block_table.shape[1], num_pages, _ptr(seq_lens), B, int(q_len),
                                  int(num_splits), _ptr(w_uv), _ptr(workspace), workspace.numel(),
                                  _ptr(out), _ptr(o_lat), _ptr(lse), e0, e1, _stream())
    _check("mla_decode_paged_out", st)
    return out, o_lat, lse


def decode_noalloc_max_bytes() -> int:
    return int(lib.mla_decode_noalloc_max_bytes())


def out_proj(d: Dims, o_lat: torch.Tensor, w_uv: torch.Tensor,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    B = o_lat.shape[0]
    H = d.n_heads
    _req(o_lat, "o_lat", torch.bfloat16, (B, H, d.d_c))
    _req(w_uv, "w_uv", torch.bfloat16, (H, d.d_c, d.d_v))
    if out is None:
        out = torch.empty((B, H, d.d_v), dtype=torch.bfloat16, device=o_lat.device)
    _req(out, "out", torch.bfloat16, (B, H, d.d_v))
    _check("mla_out_proj", lib.mla_out_proj(ctypes.byref(d), _ptr(o_lat), _ptr(w_uv), B, _ptr(out),
                                            _stream()))
    return out


def cache_bytes_per_token(d: Dims) -> int:
    return int(lib.mla_cache_bytes_per_token(ctypes.byref(d)))


def prefill_workspace_size(d: Dims, B: int, max_pages: int) -> int:
    return int(lib.mla_prefill_workspace_size(ctypes.byref(d), int(B), int(max_pages)))


def prefill_paged(d: Dims, q_nope: torch.Tensor, q_pe: torch.Tensor, q_start: torch.Tensor,
                  max_q_len: int, pool: torch.Tensor, scales: Optional[torch.Tensor],
                  block_table: torch.Tensor, seq_lens: torch.Tensor, w_uk: torch.Tensor,
                  w_uv: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  want_lse: bool = True, events=None):
    """mla_prefill_paged: q_nope [T][H][d_nope], q_pe [T][H][d_rope], q_start [B+1]
    (device int32); returns out [T][H][d_v] and lse [T][H] (or None)."""
    H = d.n_heads
    if q_nope.dim() != 3:
        raise ValueError("q_nope must be [T][H][d_nope]")
    T = q_nope.shape[0]
    B = seq_lens.shape[0]
    _req(q_nope, "q_nope", torch.bfloat16, (T, H, d.d_nope))
    _req(q_pe, "q_pe", torch.bfloat16, (T, H, d.d_rope))
    _req(q_start, "q_start", torch.int32, (B + 1,))
    num_pages = pool.shape[0]
    if _is_fp8(d):
        _req(pool, "pool", torch.uint8, pool_shape(d, num_pages))
        _req(scales, "scales", torch.float32, (num_pages, d.page_size))
    else:
        _req(pool, "pool", torch.bfloat16, pool_shape(d, num_pages))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    _req(block_table, "block_table", torch.int32)
    _req(seq_lens, "seq_lens", torch.int32, (B,))
    _req(w_uk, "w_uk", torch.bfloat16, (H, d.d_c, d.d_nope))
    _req(w_uv, "w_uv", torch.bfloat16, (H, d.d_c, d.d_v))
    max_pages = block_table.shape[1]
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(d, B, max_pages), dtype=torch.uint8,
                                device=q_nope.device)
    _req(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((T, H, d.d_v), dtype=torch.bfloat16, device=q_nope.device)
    _req(out, "out", torch.bfloat16, (T, H, d.d_v))
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
    if lse is not None:
        _req(lse, "lse", torch.float32, (T, H))
    args = (ctypes.byref(d), _ptr(q_nope), _ptr(q_pe), _ptr(q_start), T, int(max_q_len), _ptr(pool),
            _ptr(scales), _ptr(block_table), max_pages, num_pages, _ptr(seq_lens), B, _ptr(w_uk),
            _ptr(w_uv), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse))
    if events is None:
        _check("mla_prefill_paged", lib.mla_prefill_paged(*args, _stream()))
    else:
        e0, e1 = _event_handles(events)
        _check("mla_prefill_paged_timed", lib.mla_prefill_paged_timed(*args, e0, e1, _stream()))
    return out, lse
