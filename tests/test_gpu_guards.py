"""Block-table entries outside [0, num_pages) inside a sequence's range (a
caller error the library cannot see from the host): the attention kernels
must not dereference them, and every other sequence of the call must come out
bit for bit as in a call with a clean table.  The corrupted sequence's result
is unspecified and not checked.  Covers the decode tile copies (bf16 whole
tiles and 16-token pages, the fp8 tiles and their scales) and the prefill
up-projection's row reads.  Also: seq_lens outside [0, max_pages * page_size]
decode exactly as the clamped lengths."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from workload import configs, make_inputs
from workload.torch_io import bf16_bits, i32_tensor

from gpu_util import build_cache, dims_for
from test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu


def _corrupt(bt, num_pages):
    """Sequence 0's second and fifth pages moved outside the pool, one below
    and one above it."""
    bad = bt.copy()
    bad[0, 1] = -5
    bad[0, 4] = num_pages + 1000
    return bad


@pytest.mark.parametrize("fp8,page_size", [(False, 64), (False, 16), (True, 64), (True, 16)],
                         ids=["bf16_p64", "bf16_p16", "fp8_p64", "fp8_p16"])
@pytest.mark.parametrize("num_splits", [0, 1])
def test_decode_pages_outside_the_pool(fp8, page_size, num_splits):
    wl = configs.V3.with_(name="v3_badpage", fp8=fp8, batch=3, seq_len=None, seq_lens=(700, 2048, 100),
                          page_size=page_size)
    print(f"[guards decode] fp8={fp8} page={page_size} splits={num_splits}", flush=True)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    o0, l0 = mla.decode_paged(d, q, pool, scales, t["block_table"], t["seq_lens"], num_splits=num_splits)
    bad = i32_tensor(_corrupt(inp.block_table, inp.num_pages), "cuda")
    o1, l1 = mla.decode_paged(d, q, pool, scales, bad, t["seq_lens"], num_splits=num_splits)
    out0, _, _ = mla.decode_paged_out(d, q, pool, scales, t["block_table"], t["seq_lens"], t["w_uv"],
                                      num_splits=num_splits)
    out1, _, _ = mla.decode_paged_out(d, q, pool, scales, bad, t["seq_lens"], t["w_uv"], num_splits=num_splits)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(o0)[1:], bf16_bits(o1)[1:])
    assert np.array_equal(l0.cpu().numpy()[1:], l1.cpu().numpy()[1:])
    assert np.array_equal(bf16_bits(out0)[1:], bf16_bits(out1)[1:])


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_prefill_pages_outside_the_pool(fp8):
    wl = configs.V3.with_(name="v3_badpage_pf", fp8=fp8, batch=2, n_heads=4, seq_len=None, seq_lens=(700, 300),
                          q_len=150)
    print(f"[guards prefill] fp8={fp8}", flush=True)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    out0, lse0, starts, _ = run_prefill(inp, d, cache=(pool, scales, t))
    t_bad = dict(t)
    t_bad["block_table"] = i32_tensor(_corrupt(inp.block_table, inp.num_pages), "cuda")
    out1, lse1, _, _ = run_prefill(inp, d, cache=(pool, scales, t_bad))
    rows = slice(int(starts[1]), int(starts[2]))          # sequence 1's new tokens
    assert np.array_equal(out0[rows], out1[rows])
    assert np.array_equal(lse0[rows], lse1[rows])


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("num_splits", [0, 1])
def test_decode_seq_lens_are_clamped(fp8, num_splits):
    # seq_lens are clamped to [0, max_pages * page_size]: -3 decodes as an empty
    # sequence and cap + 500 as cap, bit for bit
    wl = configs.V3.with_(name="v3_clamp", fp8=fp8, batch=3, seq_len=None, seq_lens=(64, 2048, 100))
    print(f"[guards clamp] fp8={fp8} splits={num_splits}", flush=True)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    cap = inp.block_table.shape[1] * wl.page_size
    assert cap == 2048
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    clean = i32_tensor(np.array([0, cap, 100], np.int32), "cuda")
    wild = i32_tensor(np.array([-3, cap + 500, 100], np.int32), "cuda")
    r = [mla.decode_paged(d, q, pool, scales, t["block_table"], s, num_splits=num_splits) for s in (clean, wild)]
    p = [mla.decode_paged_out(d, q, pool, scales, t["block_table"], s, t["w_uv"], num_splits=num_splits,
                              want_o_lat=True, want_lse=True) for s in (clean, wild)]
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(r[0][0]), bf16_bits(r[1][0]))
    assert np.array_equal(r[0][1].cpu().numpy(), r[1][1].cpu().numpy())
    for a, b in zip(p[0], p[1]):
        if a.dtype == torch.bfloat16:
            assert np.array_equal(bf16_bits(a), bf16_bits(b))
        else:
            assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
    assert np.all(bf16_bits(r[1][0])[0] == 0) and np.all(np.isneginf(r[1][1].cpu().numpy()[0]))
