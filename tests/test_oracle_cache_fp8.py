"""Pins for the cache-size closed forms (against figures printed on the pages,
tests/golden/cache_size.json) and the per-token fp8 row quantiser (CPU only)."""
import json
import os

import numpy as np

from oracle import (cache_rows, e4m3fn_decode, fp8_quantize_rows, mha_cache_elements_per_token,
                    mla_cache_bytes_per_token, mla_cache_elements_per_token)
from workload import configs, make_inputs


def test_cache_size_against_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cache_size.json")))
    r1 = g["r1_kv_per_token"]
    per_layer = mla_cache_bytes_per_token(r1["d_c"], r1["d_rope"], fp8=False)
    assert per_layer == 1152
    total_kb = per_layer * r1["layers"] / 1024.0
    assert round(total_kb, 1) == r1["printed_kb"]              # 68.625 KiB -> "68.6KB"
    mha = g["mha_elements_row"]
    assert mha_cache_elements_per_token(mha["layers"], mha["n_heads"], mha["head_dim"]) \
        == mha["printed_elements"]
    # MLA (latent + RoPE key) vs MHA with 128 heads x 128 dims: 56.9x fewer elements
    mla = mla_cache_elements_per_token(1, 512, 64)
    assert mla == 576
    assert round(mha["printed_elements"] / mla, 1) == 56.9
    # fp8 row + one fp32 scale
    assert mla_cache_bytes_per_token(512, 64, fp8=True) == 580


def test_fp8_row_quantiser_properties():
    rng = np.random.default_rng(7)
    rows = (rng.standard_normal((300, 576)) * rng.uniform(0.01, 100, (300, 1))).astype(np.float32)
    rows[5] = 0.0
    codes, scale = fp8_quantize_rows(rows)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    absmax = np.abs(rows).max(-1)
    assert np.array_equal(scale, (absmax / np.float32(448)).astype(np.float32))
    assert scale[5] == 0 and np.all(codes[5] == 0)
    deq = e4m3fn_decode(codes) * scale[:, None].astype(np.float64)
    x = rows.astype(np.float64)
    # within half a unit in the last place: 2^-4 relative for normals,
    # 2^-10 * scale absolute in the subnormal range
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)
    # the largest element of each nonzero row lands on (or next to) the top code
    top = np.abs(e4m3fn_decode(codes)).max(-1)
    assert np.all(top[np.arange(300) != 5] >= 416)


def test_fp8_cache_rows_close_to_bf16_rows():
    wl = configs.TINY.with_(fp8=True)
    inp = make_inputs(wl)
    pos = inp.positions()
    C8, K8 = cache_rows(inp.c_kv, inp.k_pe, pos, wl.rope_base, True)
    C, K = cache_rows(inp.c_kv, inp.k_pe, pos, wl.rope_base, False)
    assert np.abs(C8 - C).max() <= 2.0 ** -4 * np.abs(C).max()
    assert np.abs(K8 - K).max() <= 2.0 ** -4 * np.abs(np.concatenate([C, K], -1)).max()
