"""mla_append_latent on the GPU: bit-exact page placement, RoPE against the
oracle, fp8 codes and scales bitwise against the oracle's encoder, and
out-of-range inputs skipped without touching memory."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import fp8_cache_codes, rope, bf16_bits_to_f64
from workload import configs, f32_to_bf16_bits, make_inputs
from workload.torch_io import bf16_bits, i32_tensor

from gpu_util import BF16_NAN, FP8_NAN, DEV, build_cache, dims_for

pytestmark = pytest.mark.gpu

V2_SMALL = configs.V2LITE.with_(name="v2small", batch=3, n_heads=16, seq_len=None,
                                seq_lens=(1, 100, 257))
V2_SMALL_P16 = V2_SMALL.with_(name="v2small_p16", page_size=16)
CASES = [configs.TINY, V2_SMALL, V2_SMALL_P16]


def _slots(inp):
    """(page, slot) of every cached token, in token order."""
    ps = inp.wl.page_size
    pos = inp.positions()
    sid = inp.seq_ids()
    pages = inp.block_table[sid, pos // ps]
    return pages, pos % ps


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_raw_placement_is_bit_exact(wl):
    inp = make_inputs(wl)
    d = dims_for(wl)
    print(f"[append raw] {wl.name}", flush=True)
    pool, _, _ = build_cache(inp, d, rope=False)
    host = bf16_bits(pool)
    pages, slots = _slots(inp)
    want = np.concatenate([inp.c_kv, inp.k_pe], axis=1)
    assert np.array_equal(host[pages, slots], want)
    written = np.zeros(host.shape[:2], bool)
    written[pages, slots] = True
    assert np.all(host[~written] == BF16_NAN)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_rope_rows_match_oracle(wl):
    inp = make_inputs(wl)
    d = dims_for(wl)
    print(f"[append rope] {wl.name}", flush=True)
    pool, _, _ = build_cache(inp, d, rope=True)
    host = bf16_bits(pool)
    pages, slots = _slots(inp)
    rows = host[pages, slots]
    assert np.array_equal(rows[:, :wl.d_c], inp.c_kv)
    kr = rope(bf16_bits_to_f64(inp.k_pe), inp.positions(), wl.rope_base)
    want = f32_to_bf16_bits(kr.astype(np.float32))
    got = rows[:, wl.d_c:]
    mism = np.mean(got != want)
    assert mism <= 1e-3, mism
    err = np.abs(bf16_bits_to_f64(got) - kr)
    assert np.all(err <= 2.0 ** -8 * np.abs(kr) + 1e-30)


@pytest.mark.parametrize("wl", [configs.TINY.with_(fp8=True), V2_SMALL.with_(fp8=True),
                                V2_SMALL_P16.with_(fp8=True)], ids=lambda w: w.name + "_fp8")
def test_fp8_codes_and_scales_match_oracle(wl):
    inp = make_inputs(wl)
    d = dims_for(wl)
    print(f"[append fp8] {wl.name}", flush=True)
    pool, scales, _ = build_cache(inp, d, rope=True)
    host = pool.cpu().numpy()
    hs = scales.cpu().numpy()
    pages, slots = _slots(inp)
    codes, scale = fp8_cache_codes(inp.c_kv, inp.k_pe, inp.positions(), wl.rope_base)
    got = host[pages, slots]
    n_bad = int(np.sum(got != codes))
    assert n_bad <= max(1, int(1e-5 * codes.size)), n_bad
    assert int(np.sum(hs[pages, slots].view(np.uint32) != scale.view(np.uint32))) <= 1
    written = np.zeros(host.shape[:2], bool)
    written[pages, slots] = True
    assert np.all(host[~written] == FP8_NAN)
    assert np.all(np.isnan(hs[~written]))


def test_out_of_range_tokens_are_skipped():
    wl = configs.TINY
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, _ = mla.new_pool(d, inp.num_pages, DEV)
    pool.view(torch.int16).fill_(BF16_NAN)
    bt = inp.block_table.copy()
    bt[0, 1] = inp.num_pages + 5          # page id outside the pool
    T = 6
    c = torch.ones((T, wl.d_c), dtype=torch.bfloat16, device=DEV)
    k = torch.ones((T, wl.d_rope), dtype=torch.bfloat16, device=DEV)
    positions = i32_tensor(np.array([20, 3, 1000, -1, 5, 0]), DEV)   # 20 -> bad page; 1000 -> past table
    seq_ids = i32_tensor(np.array([0, 7, 1, 0, -2, 1]), DEV)        # 7, -2 -> no such sequence
    mla.append_latent(d, c, k, positions, seq_ids, i32_tensor(bt, DEV), pool, None, rope=False)
    host = bf16_bits(pool)
    written = np.argwhere(np.any(host != BF16_NAN, axis=-1))
    want = {(int(bt[1, 0]), 0)}            # only the last token (seq 1, position 0) is valid
    assert {tuple(x) for x in written} == want
