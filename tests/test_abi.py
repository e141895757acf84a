"""The C ABI on the host (CPU only): the library loads, exports every symbol
include/mla.h declares, and rejects bad host arguments before enqueueing
anything.  Every call here fails validation (asserted), so no kernel is ever
launched with the placeholder pointers used below."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_nope_amd as mla
from mla_latent_kv_nope_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib = _native.lib
VALIDATION_ERRORS = (_native.MLA_ERR_INVALID_ARG, _native.MLA_ERR_UNSUPPORTED,
                     _native.MLA_ERR_WORKSPACE)
P = 0x100000  # aligned placeholder; never dereferenced (validation fails first)


def header_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert set(names) == set(_native.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_dims_struct_layout():
    assert ctypes.sizeof(_native.Dims) == 40
    assert _native.Dims.rope_base.offset == 32


def test_status_strings():
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_ARG"), (2, "MLA_ERR_UNSUPPORTED"),
                       (3, "MLA_ERR_WORKSPACE"), (4, "MLA_ERR_HIP")]:
        assert mla.status_string(code) == name
    assert mla.status_string(99) == "MLA_ERR_UNKNOWN"


def test_cache_bytes_per_token():
    assert mla.cache_bytes_per_token(mla.make_dims(128, 512, 64, 128, 128, 64)) == 1152
    assert mla.cache_bytes_per_token(mla.make_dims(128, 512, 64, 128, 128, 64, fp8=True)) == 580
    assert mla.cache_bytes_per_token(mla.make_dims(4, 32, 16, 16, 16, 16)) == 96
    assert lib.mla_cache_bytes_per_token(None) == 0


def test_workspace_size():
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    n = lib.mla_decode_workspace_size(ctypes.byref(d), 64, 256)
    # plan (66 int32) + partial O (bf16) and lse (fp32) for 256 + 64 slots,
    # 256-byte aligned pieces
    assert n >= (256 + 64) * 128 * (512 * 2 + 4)
    assert n < (256 + 64) * 128 * (512 * 2 + 4) + 4096
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 0, 256) == 0
    bad = mla.make_dims(128, 256, 64, 128, 128, 64)
    assert lib.mla_decode_workspace_size(ctypes.byref(bad), 4, 8) == 0


def _expect(code, want):
    assert code in VALIDATION_ERRORS, code
    assert code == want, (mla.status_string(code), mla.status_string(want))


def test_append_validation():
    d = mla.make_dims(4, 32, 16, 16, 16, 16)
    f = lib.mla_append_latent
    _expect(f(None, P, P, P, P, P, 2, 4, 10, 5, P, None, 0, None), _native.MLA_ERR_INVALID_ARG)
    _expect(f(ctypes.byref(d), None, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_INVALID_ARG)
    _expect(f(ctypes.byref(d), P, P, P, P, P, 2, 4, 10, -1, P, None, 0, None),
            _native.MLA_ERR_INVALID_ARG)
    _expect(f(ctypes.byref(d), P, P, P, P, P, 2, 4, 10, 5, P, None, 7, None),
            _native.MLA_ERR_INVALID_ARG)                                  # unknown flag
    _expect(f(ctypes.byref(d), P + 2, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_INVALID_ARG)                                  # misaligned c_kv
    _expect(f(ctypes.byref(d), P, P, P, P, P, 2, 4, 10, 5, P, P, 0, None),
            _native.MLA_ERR_INVALID_ARG)                                  # scales on bf16
    d8 = mla.make_dims(4, 32, 16, 16, 16, 16, fp8=True)
    _expect(f(ctypes.byref(d8), P, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_INVALID_ARG)                                  # fp8 without scales
    odd_ps = mla.make_dims(4, 32, 16, 16, 16, 24)
    _expect(f(ctypes.byref(odd_ps), P, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_UNSUPPORTED)
    neg_scale = mla.make_dims(4, 32, 16, 16, 16, 16, softmax_scale=-0.5)
    _expect(f(ctypes.byref(neg_scale), P, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_INVALID_ARG)
    odd_dims = mla.make_dims(4, 64, 16, 16, 16, 16)
    _expect(f(ctypes.byref(odd_dims), P, P, P, P, P, 2, 4, 10, 5, P, None, 0, None),
            _native.MLA_ERR_UNSUPPORTED)
    # zero tokens is a no-op that succeeds without touching anything
    assert f(ctypes.byref(d), None, None, None, None, None, 2, 4, 10, 0, None, None, 0, None) == 0


def test_absorb_and_out_proj_validation():
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    _expect(lib.mla_absorb_q(ctypes.byref(d), P, P, P, P, 0, P, None), _native.MLA_ERR_INVALID_ARG)
    _expect(lib.mla_absorb_q(ctypes.byref(d), P, P, None, P, 4, P, None),
            _native.MLA_ERR_INVALID_ARG)
    _expect(lib.mla_absorb_q(ctypes.byref(d), P, P, P, P + 8, 4, P, None),
            _native.MLA_ERR_INVALID_ARG)
    too_many = mla.make_dims(129, 512, 64, 128, 128, 64)
    _expect(lib.mla_absorb_q(ctypes.byref(too_many), P, P, P, P, 4, P, None),
            _native.MLA_ERR_UNSUPPORTED)
    _expect(lib.mla_out_proj(ctypes.byref(d), P, None, 4, P, None), _native.MLA_ERR_INVALID_ARG)
    _expect(lib.mla_out_proj(ctypes.byref(d), P, P, -3, P, None), _native.MLA_ERR_INVALID_ARG)


def test_decode_validation():
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_decode_paged
    need = lib.mla_decode_workspace_size(ctypes.byref(d), 4, 8)
    args = dict(q=P, pool=P, scales=None, bt=P, maxp=8, nump=40, sl=P, B=4, ns=8, ws=P, wsb=need,
                o=P, lse=P)

    def call(**kw):
        a = dict(args, **kw)
        return f(ctypes.byref(d), a["q"], a["pool"], a["scales"], a["bt"], a["maxp"], a["nump"],
                 a["sl"], a["B"], a["ns"], a["ws"], a["wsb"], a["o"], a["lse"], None)

    # fp8 caches decode only with the 576-element rows (d_c 512 + d_rope 64)
    d8 = mla.make_dims(128, 512, 64, 128, 128, 64, fp8=True)
    assert lib.mla_decode_workspace_size(ctypes.byref(d8), 4, 8) == need
    t8 = mla.make_dims(4, 32, 16, 16, 16, 16, fp8=True)
    assert lib.mla_decode_workspace_size(ctypes.byref(t8), 4, 8) == 0
    _expect(f(ctypes.byref(t8), P, P, P, P, 8, 40, P, 4, 8, P, need, P, P, None),
            _native.MLA_ERR_UNSUPPORTED)
    _expect(f(ctypes.byref(d8), P, P, None, P, 8, 40, P, 4, 8, P, need, P, P, None),
            _native.MLA_ERR_INVALID_ARG)                          # fp8 without scales
    _expect(call(wsb=need - 1), _native.MLA_ERR_WORKSPACE)
    _expect(call(ws=P + 16), _native.MLA_ERR_INVALID_ARG)         # workspace not 256-aligned
    _expect(call(q=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(B=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(ns=-1), _native.MLA_ERR_INVALID_ARG)
    _expect(call(scales=P), _native.MLA_ERR_INVALID_ARG)         # scales with a bf16 cache
    _expect(call(maxp=0), _native.MLA_ERR_INVALID_ARG)


def test_decode_noalloc_validation():
    """mla_decode_paged_noalloc: same argument checks as the decode calls (no
    workspace argument), and a required workspace above the library's device
    array is MLA_ERR_WORKSPACE, both before any HIP call."""
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_decode_paged_noalloc
    cap = lib.mla_decode_noalloc_max_bytes()
    assert cap == 64 << 20

    def call(B=4, q_len=1, ns=8, q=P, o=P, scales=None):
        return f(ctypes.byref(d), q, P, scales, P, 8, 40, P, B, q_len, ns, o, P, None)

    _expect(call(q=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(o=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q=P + 8), _native.MLA_ERR_INVALID_ARG)
    _expect(call(B=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q_len=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(scales=P), _native.MLA_ERR_INVALID_ARG)
    # the largest batch that fits the array, and one more query sequence
    B = 1
    while lib.mla_decode_workspace_size(ctypes.byref(d), B + 1, 8) <= cap:
        B += 1
    assert lib.mla_decode_workspace_size(ctypes.byref(d), B + 1, 8) > cap
    _expect(call(B=B + 1), _native.MLA_ERR_WORKSPACE)
    _expect(call(B=(B + 1) // 2 + 1, q_len=2), _native.MLA_ERR_WORKSPACE)


def test_decode_multi_validation():
    """mla_decode_paged_multi: q_len range, and a workspace sized for B * q_len
    query sequences."""
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_decode_paged_multi
    B, ql = 4, 3
    need = lib.mla_decode_workspace_size(ctypes.byref(d), B * ql, 0)
    assert need > lib.mla_decode_workspace_size(ctypes.byref(d), B, 0)

    def call(q_len=ql, wsb=need, q=P):
        return f(ctypes.byref(d), q, P, None, P, 8, 40, P, B, q_len, 0, P, wsb, P, P, None)

    for bad in (0, -1, _native.MLA_MAX_Q_LEN + 1):
        _expect(call(q_len=bad), _native.MLA_ERR_INVALID_ARG)
    _expect(call(wsb=need - 1), _native.MLA_ERR_WORKSPACE)
    _expect(call(q=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q=P + 8), _native.MLA_ERR_INVALID_ARG)          # q not 16-byte aligned


def test_decode_out_validation():
    """mla_decode_paged_out: out and w_uv required, o_lat and lse optional,
    the fused merge exists for d_c 512 / d_v 128 only."""
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_decode_paged_out
    B, ql = 4, 2
    need = lib.mla_decode_workspace_size(ctypes.byref(d), B * ql, 0)

    def call(dims=d, q=P, w=P, wsb=need, out=P, o=None, lse=None, q_len=ql, B=B):
        return f(ctypes.byref(dims), q, P, None, P, 8, 40, P, B, q_len, 0, w, P, wsb, out, o, lse,
                 None, None, None)

    _expect(call(out=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(w=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(out=P + 8), _native.MLA_ERR_INVALID_ARG)         # out not 16-byte aligned
    _expect(call(w=P + 8), _native.MLA_ERR_INVALID_ARG)           # w_uv not 16-byte aligned
    _expect(call(o=P + 8), _native.MLA_ERR_INVALID_ARG)           # o_lat not 16-byte aligned
    _expect(call(lse=P + 2), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q_len=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(B=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(wsb=need - 1), _native.MLA_ERR_WORKSPACE)
    tiny = mla.make_dims(4, 32, 16, 16, 16, 16)
    _expect(call(dims=tiny, wsb=1 << 30), _native.MLA_ERR_UNSUPPORTED)


def test_append_absorb_validation():
    """mla_append_absorb checks both argument sets as the separate calls do."""
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_append_absorb

    def call(c_kv=P, T=5, flags=0, q_nope=P, B=4, w_uk=P, scales=None, dims=d, q_out=P):
        return f(ctypes.byref(dims), c_kv, P, P, P, P, 4, 8, 40, T, P, scales, flags,
                 q_nope, P, P, w_uk, B, q_out, None)

    _expect(call(c_kv=None), _native.MLA_ERR_INVALID_ARG)        # append side
    _expect(call(c_kv=P + 2), _native.MLA_ERR_INVALID_ARG)
    _expect(call(T=-1), _native.MLA_ERR_INVALID_ARG)
    _expect(call(flags=7), _native.MLA_ERR_INVALID_ARG)
    _expect(call(scales=P), _native.MLA_ERR_INVALID_ARG)         # scales with a bf16 cache
    _expect(call(q_nope=None), _native.MLA_ERR_INVALID_ARG)      # absorb side
    _expect(call(B=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(w_uk=P + 8), _native.MLA_ERR_INVALID_ARG)
    _expect(call(q_out=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(T=0, B=0), _native.MLA_ERR_INVALID_ARG)         # nothing to append, still absorbs
    _expect(call(dims=mla.make_dims(129, 512, 64, 128, 128, 64)), _native.MLA_ERR_UNSUPPORTED)


def test_binding_rejects_host_tensors():
    import torch
    d = mla.make_dims(4, 32, 16, 16, 16, 16)
    with pytest.raises(ValueError):
        mla.out_proj(d, torch.zeros(2, 4, 32, dtype=torch.bfloat16),
                     torch.zeros(4, 32, 16, dtype=torch.bfloat16))


def test_single_hip_runtime_in_process():
    # libmla must bind the HIP runtime PyTorch brought in, not a second copy
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip


def test_project_append_validation():
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_project_append
    T, dm = 8, 7168
    need = lib.mla_project_append_workspace_size(ctypes.byref(d), dm, T)
    assert need == 4 * ((dm // 256 + 3) // 4) * T * 576   # fp32 partials, one per run of four 256-chunks
    assert lib.mla_project_append_workspace_size(ctypes.byref(d), 7000, T) == 0   # not a multiple of 256
    t = mla.make_dims(4, 32, 16, 16, 16, 16)                                     # 48-wide rows
    assert lib.mla_project_append_workspace_size(ctypes.byref(t), 256, T) == 0

    def call(dm=dm, h=P, ws=P, wsb=need, T=T, dims=d):
        return f(ctypes.byref(dims), dm, h, P, P, P, P, 4, 8, 40, T, P, None, ws, wsb, None)

    _expect(call(dm=7000), _native.MLA_ERR_UNSUPPORTED)
    _expect(call(dims=t, dm=256), _native.MLA_ERR_UNSUPPORTED)
    _expect(call(dm=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(wsb=need - 1), _native.MLA_ERR_WORKSPACE)
    _expect(call(ws=P + 16), _native.MLA_ERR_INVALID_ARG)        # workspace not 256-aligned
    _expect(call(h=None), _native.MLA_ERR_INVALID_ARG)
    assert call(T=0) == _native.MLA_OK                           # no tokens: nothing enqueued


def test_prefill_validation():
    d = mla.make_dims(128, 512, 64, 128, 128, 64)
    f = lib.mla_prefill_paged
    B, mp = 2, 4
    need = lib.mla_prefill_workspace_size(ctypes.byref(d), B, mp)
    # K_nope and V^T: B * H * 128 tokens-padded-to-32 bf16 each, then the
    # RoPE keys B * 64 per token
    assert need == 2 * B * 128 * 128 * (mp * 64) * 2 + B * 64 * (mp * 64) * 2
    p16 = mla.make_dims(4, 512, 64, 128, 128, 16)
    assert lib.mla_prefill_workspace_size(ctypes.byref(p16), 1, 3) == \
        2 * 4 * 128 * 64 * 2 + 64 * 64 * 2                                  # 48 -> 64 tokens
    tiny = mla.make_dims(4, 32, 16, 16, 16, 16)
    assert lib.mla_prefill_workspace_size(ctypes.byref(tiny), B, mp) == 0
    d8 = mla.make_dims(128, 512, 64, 128, 128, 64, fp8=True)
    assert lib.mla_prefill_workspace_size(ctypes.byref(d8), B, mp) == need

    def call(dims=d, T=16, mq=16, qn=P, ws=P, wsb=need, B=B, lse=None, qs=P, sc=None):
        return f(ctypes.byref(dims), qn, P, qs, T, mq, P, sc, P, mp, 40, P, B, P, P, ws, wsb, P,
                 lse, None)

    _expect(call(dims=tiny), _native.MLA_ERR_UNSUPPORTED)
    _expect(call(dims=d8), _native.MLA_ERR_INVALID_ARG)             # fp8 without scales
    _expect(call(sc=P), _native.MLA_ERR_INVALID_ARG)                # scales with a bf16 cache
    _expect(call(T=-1), _native.MLA_ERR_INVALID_ARG)
    _expect(call(mq=-1), _native.MLA_ERR_INVALID_ARG)
    _expect(call(B=0), _native.MLA_ERR_INVALID_ARG)
    _expect(call(qn=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(qs=None), _native.MLA_ERR_INVALID_ARG)
    _expect(call(qn=P + 8), _native.MLA_ERR_INVALID_ARG)          # q_nope not 16-byte aligned
    _expect(call(lse=P + 2), _native.MLA_ERR_INVALID_ARG)
    _expect(call(ws=P + 16), _native.MLA_ERR_INVALID_ARG)         # workspace not 256-aligned
    _expect(call(wsb=need - 1), _native.MLA_ERR_WORKSPACE)
    _expect(call(mq=(1 << 24) + 1), _native.MLA_ERR_UNSUPPORTED)
    assert call(T=0) == _native.MLA_OK                            # nothing to do
    assert call(mq=0) == _native.MLA_OK
