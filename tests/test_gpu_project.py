"""mla_project_append on the GPU against the oracle: the down-projection
(`project_latent`: bf16 of the exact h . w_down^T) followed by the cached-row
content of `cache_rows`; placement bit-exact (every other slot keeps its NaN
poison).

Bar: every projected c_kv value is within half a bf16 step plus the fp32
summation bound ((d_model - 1) 2^-24 sum |h_k w_k|) of the exact value; where
that bound is below half a step (all but outputs whose terms cancel to near
zero) the value is the oracle's bf16 value or one bf16 step away (the GPU
rounds an fp32 sum, the oracle the exact value; a value whose fp32 sum falls
on the other side of a rounding midpoint moves by one step), with at most
1 % of them moved and at most 0.1 % moved more; the rotated key part meets the decode bar
(max |gpu - oracle| <= 2e-2, relative L2 <= 5e-3).  fp8 rows are compared
code by code with the oracle's encoder applied to the oracle's bf16 rows: a
value that moved one bf16 step can cross an fp8 rounding midpoint, so codes
may be the adjacent code (same sign) on at most 1 % of the elements, and each
row's scale (absmax / 448) may move by one bf16 step of its absmax.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import bf16_bits_to_f64, cache_rows, fp8_cache_codes, project_latent
from workload import configs, make_inputs, make_projection_inputs
from workload.torch_io import bf16_bits, bf16_tensor, to_device

from gpu_util import BF16_NAN, FP8_NAN, DEV, assert_close, dims_for, poison_pool

pytestmark = pytest.mark.gpu

CASES = [
    # (workload giving the paging and positions, d_model)
    (configs.V3.with_(name="v3_t3", batch=3, seq_len=None, seq_lens=(1, 1, 1)), 256),
    (configs.V3.with_(name="v3_t64", batch=4, seq_len=None, seq_lens=(16, 16, 16, 16)), 7168),
    (configs.V3.with_(name="v3_t70_p16", batch=3, seq_len=None, seq_lens=(33, 2, 35), page_size=16), 768),
    (configs.V2LITE.with_(name="v2_t5", batch=2, seq_len=None, seq_lens=(2, 3)), 2048),
    (configs.V3.with_(name="v3_fp8_t64", batch=2, seq_len=None, seq_lens=(40, 24), fp8=True), 7168),
    (configs.V3.with_(name="v3_t20_p256", batch=2, seq_len=None, seq_lens=(12, 8), page_size=256), 512),
]


def _run(wl, d_model):
    inp = make_inputs(wl)
    T, R = inp.total_tokens, wl.d_latent
    pin = make_projection_inputs(T, d_model, R, seed=5)
    d = dims_for(wl)
    t = to_device(inp, DEV)
    pool, scales = mla.new_pool(d, inp.num_pages, DEV)
    poison_pool(pool, scales)
    mla.project_append(d, bf16_tensor(pin.h, DEV), bf16_tensor(pin.w_down, DEV), t["positions"],
                       t["seq_ids"], t["block_table"], pool, scales)
    torch.cuda.synchronize()
    ps = wl.page_size
    pos, sid = inp.positions(), inp.seq_ids()
    pages, slots = inp.block_table[sid, pos // ps], pos % ps
    return inp, pin, pool, scales, pages, slots


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0].name}_dm{c[1]}")
def test_project_append_matches_oracle(case):
    wl, d_model = case
    print(f"[project append] {wl.name} d_model={d_model}", flush=True)
    inp, pin, pool, scales, pages, slots = _run(wl, d_model)
    c_bits, k_bits = project_latent(pin.h, pin.w_down, wl.d_c)
    C, Kr = cache_rows(c_bits, k_bits, inp.positions(), wl.rope_base, wl.fp8)
    if not wl.fp8:
        host = bf16_bits(pool)
        rows = host[pages, slots]
        got_c = rows[:, :wl.d_c].astype(np.int32)
        want_c = c_bits.astype(np.int32)
        step = np.abs(got_c - want_c)
        same_sign = (got_c >> 15) == (want_c >> 15)
        # fp32 accumulation of d_model exact bf16 products, in any order, is
        # within (d_model - 1) u sum |h_k w_k| (u = 2^-24) of the exact sum;
        # rounding to bf16 adds half a step.  Where that error is below half
        # a step the result is the exact value rounded (step <= 1); near-zero
        # outputs, where the terms cancel, may be further off within it.
        h64, w64 = bf16_bits_to_f64(pin.h), bf16_bits_to_f64(pin.w_down)
        y = h64 @ w64.T
        bound = (d_model - 1) * 2.0 ** -24 * (np.abs(h64) @ np.abs(w64).T)
        got_v = bf16_bits_to_f64(rows[:, :wl.d_c])
        err = np.abs(got_v - y[:, :wl.d_c])
        # half a bf16 step at the larger of the two magnitudes: |x| in
        # [2^(E-1), 2^E) has steps of 2^(E-8)
        _, E = np.frexp(np.maximum(np.abs(got_v), np.abs(y[:, :wl.d_c])))
        half_step = np.ldexp(1.0, E - 9)
        assert np.all(err <= half_step + bound[:, :wl.d_c]), float(np.max(err - half_step - bound[:, :wl.d_c]))
        well = bound[:, :wl.d_c] < half_step
        assert np.all(((step == 0) | ((step == 1) & same_sign))[well]), int(step[well].max())
        assert np.mean(step) <= 1e-2, np.mean(step)
        assert np.mean(step > 1) <= 1e-3, np.mean(step > 1)
        assert_close(bf16_bits_to_f64(rows[:, wl.d_c:]), Kr, "k_pe (rotated)")
        written = np.zeros(host.shape[:2], bool)
        written[pages, slots] = True
        assert np.all(host[~written] == BF16_NAN)
    else:
        host = pool.cpu().numpy()
        hs = scales.cpu().numpy()
        codes, scale = fp8_cache_codes(c_bits, k_bits, inp.positions(), wl.rope_base)
        got = host[pages, slots].astype(np.int32)
        want = codes.astype(np.int32)
        same_sign = (got & 0x80) == (want & 0x80)
        assert np.all(same_sign | ((got & 0x7F) == 0) | ((want & 0x7F) == 0))
        step = np.abs((got & 0x7F) - (want & 0x7F))
        assert step.max() <= 1 and np.mean(step) <= 1e-2, (int(step.max()), float(np.mean(step)))
        rel = np.abs(hs[pages, slots].astype(np.float64) / scale.astype(np.float64) - 1.0)
        assert rel.max() <= 2.0 ** -8, rel.max()
        written = np.zeros(host.shape[:2], bool)
        written[pages, slots] = True
        assert np.all(host[~written] == FP8_NAN) and np.all(np.isnan(hs[~written]))


def test_project_append_equals_append_of_projected_rows():
    # the fused call stores exactly what mla_append_latent stores for the
    # same bf16 rows: projection computed on the GPU, rounded rows read back
    wl, d_model = CASES[1]
    inp, pin, pool, _, pages, slots = _run(wl, d_model)
    d = dims_for(wl)
    rows = bf16_bits(pool)[pages, slots]
    t = to_device(inp, DEV)
    # k_pe before rotation is not stored; recompute rows through the plain
    # append from the stored c_kv and the oracle's (identical up to one step)
    # un-rotated key, then compare only the c_kv half, which append copies
    pool2, _ = mla.new_pool(d, inp.num_pages, DEV)
    poison_pool(pool2, None)
    _, k_bits = project_latent(pin.h, pin.w_down, wl.d_c)
    mla.append_latent(d, bf16_tensor(np.ascontiguousarray(rows[:, :wl.d_c]), DEV),
                      bf16_tensor(k_bits, DEV), t["positions"], t["seq_ids"], t["block_table"], pool2)
    torch.cuda.synchronize()
    rows2 = bf16_bits(pool2)[pages, slots]
    assert np.array_equal(rows2[:, :wl.d_c], rows[:, :wl.d_c])
