"""A cache pool larger than 4 GiB, with every other block-table entry moved to
a page that starts past the 4 GiB mark: the append's scatter, the decode
kernel's tile copies (bf16 rows, fp8 codes and their per-token scales) and
the prefill reads must all form page addresses in 64 bits.  Same bar as the
other parity tests: max |gpu - oracle| <= 2e-2 and relative L2 <= 5e-3.
"""
import numpy as np
import pytest

import mla_latent_kv_nope_amd as mla
from oracle import reference_decode
from workload import configs, make_inputs
from workload.torch_io import i32_tensor, to_device

from gpu_util import DEV, assert_close, decode_step, dims_for, poison_pool
from test_gpu_prefill import compare, run_prefill

pytestmark = pytest.mark.gpu

FOUR_GIB = 4 << 30


def big_pool_cache(inp, d):
    """Pool of (first page past 4 GiB) + inp.num_pages pages; block-table
    entries in odd columns move up by that first page's index."""
    wl = inp.wl
    row_bytes = (wl.d_c + wl.d_rope) * (1 if wl.fp8 else 2)
    hi0 = FOUR_GIB // (row_bytes * wl.page_size) + 1
    num_pages = hi0 + inp.num_pages
    bt = inp.block_table.copy()
    moved = (bt >= 0) & (np.arange(bt.shape[1])[None, :] % 2 == 1)
    bt[moved] += hi0
    assert moved.any() and (~moved & (bt >= 0)).any()
    print(f"[big pool] {wl.name}: {num_pages} pages, {num_pages * row_bytes * wl.page_size / 2**30:.4f} GiB, "
          f"{int(moved.sum())} pages past 4 GiB", flush=True)
    t = to_device(inp, DEV)
    t["block_table"] = i32_tensor(bt, DEV)
    pool, scales = mla.new_pool(d, num_pages, DEV)
    poison_pool(pool, scales)
    mla.append_latent(d, t["c_kv"], t["k_pe"], t["positions"], t["seq_ids"], t["block_table"],
                      pool, scales)
    return pool, scales, t


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("num_splits", [0, 1])
def test_decode_with_pages_past_4gib(fp8, num_splits):
    wl = configs.V3.with_(name=f"v3_bigpool_{'fp8' if fp8 else 'bf16'}", fp8=fp8, batch=3, seq_len=None,
                          seq_lens=(700, 2048, 33))
    inp = make_inputs(wl)
    d = dims_for(wl)
    res = decode_step(inp, d, num_splits=num_splits, cache=big_pool_cache(inp, d))
    ref = reference_decode(inp)
    assert_close(res["out"], ref["out"], "out")
    assert_close(res["o_lat"], ref["o_lat"], "o_lat")
    assert np.max(np.abs(res["lse"] - ref["lse"])) <= 1e-2


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_prefill_with_pages_past_4gib(fp8):
    wl = configs.V3.with_(name=f"v3_bigpool_pf_{'fp8' if fp8 else 'bf16'}", fp8=fp8, batch=2, n_heads=4,
                          seq_len=None, seq_lens=(700, 300), q_len=150)
    inp = make_inputs(wl)
    d = dims_for(wl)
    out, lse, starts, _ = run_prefill(inp, d, cache=big_pool_cache(inp, d))
    compare(inp, out, lse, starts)
