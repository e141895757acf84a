"""mla_decode_paged_out (decode with the W_UV projection in the merge kernel)
on the GPU.

Checks, on the same seeded inputs and split count:
  * o_lat and lse bit-equal to mla_decode_paged_multi (the merge arithmetic is
    the same; a sequence held by one piece is merged from its bf16 partial with
    weight 1, which reproduces the row the split kernel writes directly);
  * out against mla_out_proj applied to that o_lat: the same bf16 operands,
    only the order of the fp32 additions differs, so within 2^-7 relative of
    the largest |out| element (a few bf16 steps);
  * out, o_lat and lse against the fp64 oracle at the bar
    (max |gpu - oracle| <= 2e-2, ||gpu - oracle|| / ||oracle|| <= 5e-3).
Covers several row blocks of 32 sequences with a ragged last block, empty
sequences, heads not a multiple of 8, the fp8 cache and q_len > 1.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import reference_decode, reference_decode_multi
from workload import configs, make_inputs
from workload.torch_io import bf16_bits, i32_tensor

from gpu_util import DEV, assert_close, build_cache, dims_for

pytestmark = pytest.mark.gpu

CASES = [
    configs.V3.with_(name="v3_small", batch=5, seq_len=None, seq_lens=(1, 31, 32, 33, 1500)),
    # 70 sequences: row blocks of 32, 32 and 6
    configs.V3.with_(name="v3_b70", batch=70, seq_len=None,
                     seq_lens=tuple(int(x) for x in np.arange(70) * 37 % 401 + 1)),
    configs.V3.with_(name="v3_h40", batch=3, n_heads=40, seq_len=None, seq_lens=(64, 77, 1)),
    configs.V3.with_(name="v3_h3", batch=2, n_heads=3, seq_len=None, seq_lens=(700, 2)),
    configs.V3.with_(name="v3_fp8", fp8=True, batch=5, seq_len=None, seq_lens=(1, 31, 33, 1500, 64)),
    configs.V2LITE.with_(name="v2lite_ragged", seq_len=None, seq_lens=tuple(range(1, 161, 10))),
    configs.V3.with_(name="v3_q2", batch=3, seq_len=None, seq_lens=(2, 65, 1500), q_len=2),
    configs.V3.with_(name="v3_fp8_q3", fp8=True, batch=2, seq_len=None, seq_lens=(5, 800), q_len=3),
]


def _absorbed(inp, d, t):
    wl = inp.wl
    B, ql, H = wl.batch, wl.q_len, wl.n_heads
    qn = t["q_nope"].reshape(B * ql, H, wl.d_nope)
    qp = t["q_pe"].reshape(B * ql, H, wl.d_rope)
    q = mla.absorb_q(d, qn, qp, t["q_pos"].reshape(B * ql).contiguous(), t["w_uk"])
    return q.view(B, ql, H, wl.d_latent)


def _f(x):
    return x.float().cpu().numpy().astype(np.float64)


def _bits_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("num_splits", [1, 3, 0])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_decode_out_matches_decode_then_out_proj(wl, num_splits):
    inp = make_inputs(wl)
    d = dims_for(wl)
    B, ql, H = wl.batch, wl.q_len, wl.n_heads
    print(f"[decode_out] {wl.name} splits={num_splits} seq_lens={list(inp.seq_lens)[:8]}", flush=True)
    pool, scales, t = build_cache(inp, d)
    q = _absorbed(inp, d, t)
    o_ref, l_ref = mla.decode_paged_multi(d, q, pool, scales, t["block_table"], t["seq_lens"],
                                          num_splits=num_splits)
    out_ref = mla.out_proj(d, o_ref.view(B * ql, H, wl.d_c), t["w_uv"]).view(B, ql, H, wl.d_v)
    out, o_lat, lse = mla.decode_paged_out(d, q, pool, scales, t["block_table"], t["seq_lens"], t["w_uv"],
                                           num_splits=num_splits, want_o_lat=True, want_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(o_lat), bf16_bits(o_ref))
    assert np.array_equal(lse.cpu().numpy(), l_ref.cpu().numpy())
    x, y = _f(out), _f(out_ref)
    scale = max(float(np.max(np.abs(y))), 1e-30)
    print(f"[margin] out vs out_proj: max_abs={np.max(np.abs(x - y)):.3e} (bar {scale * 2**-7:.3e})",
          flush=True)
    assert np.max(np.abs(x - y)) <= scale * 2.0 ** -7
    # oracle
    ref = reference_decode_multi(inp) if ql > 1 else reference_decode(inp)
    shp = (B, ql, H) if ql > 1 else (B, H)
    assert_close(x.reshape(shp + (wl.d_v,)), ref["out"], "out")
    assert_close(_f(o_lat).reshape(shp + (wl.d_c,)), ref["o_lat"], "o_lat")
    fin = np.isfinite(ref["lse"])
    got = lse.cpu().numpy().astype(np.float64).reshape(shp)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.max(np.abs(got[fin] - ref["lse"][fin])) <= 1e-2


def test_decode_out_optional_outputs_and_empty_sequences():
    # o_lat / lse not requested; sequences 0 and 2 empty: their out rows are 0
    wl = configs.V3.with_(name="v3_empty", batch=4, seq_len=None, seq_lens=(5, 1, 9, 70))
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    seq_lens = i32_tensor(np.array([0, 1, 0, 70]), DEV)
    out, o_lat, lse = mla.decode_paged_out(d, q, pool, scales, t["block_table"], seq_lens, t["w_uv"])
    assert o_lat is None and lse is None
    o2, ol2, l2 = mla.decode_paged_out(d, q, pool, scales, t["block_table"], seq_lens, t["w_uv"],
                                       want_o_lat=True, want_lse=True)
    o_dec, l_dec = mla.decode_paged(d, q, pool, scales, t["block_table"], seq_lens)
    torch.cuda.synchronize()
    o = _f(out)
    assert np.all(o[[0, 2]] == 0)
    assert np.array_equal(bf16_bits(out), bf16_bits(o2))
    assert np.array_equal(bf16_bits(ol2), bf16_bits(o_dec))
    assert np.array_equal(l2.cpu().numpy(), l_dec.cpu().numpy())
    assert np.all(np.isneginf(l2.cpu().numpy()[[0, 2]]))
    # one token: o_lat is its latent row, out = W_UV[h]^T c_kv[0] (fp32 sum of bf16 products)
    row = _bits_f64(inp.c_kv[inp.cu_seqlens[1]])
    want = np.einsum("c,hcv->hv", row, _bits_f64(inp.w_uv))
    assert_close(o[1], want, "out single token")


def test_decode_out_refuses_bad_arguments():
    wl = configs.TINY
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    # d_c 32: the fused merge exists for d_c 512 / d_v 128 only
    with pytest.raises(mla.MlaError) as e:
        mla.decode_paged_out(d, q, pool, scales, t["block_table"], t["seq_lens"], t["w_uv"])
    assert "UNSUPPORTED" in str(e.value)
