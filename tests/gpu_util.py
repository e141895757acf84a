"""Helpers for the GPU tests: build a paged cache through the library, run the
three decode calls, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mla_latent_kv_nope_amd as mla
from workload import unused_slots
from workload.torch_io import to_device

DEV = "cuda"
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F


def dims_for(wl, page_size=None):
    return mla.make_dims(wl.n_heads, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v,
                         page_size or wl.page_size, fp8=wl.fp8, softmax_scale=wl.softmax_scale,
                         rope_base=wl.rope_base)


def poison_pool(pool: torch.Tensor, scales):
    """Fill every slot with NaN so that reading an unwritten slot shows up."""
    if pool.dtype == torch.bfloat16:
        pool.view(torch.int16).fill_(BF16_NAN)
    else:
        pool.fill_(FP8_NAN)
    if scales is not None:
        scales.fill_(float("nan"))


def build_cache(inp, d, dev_inputs=None, poison=True, rope=True):
    t = dev_inputs or to_device(inp, DEV)
    pool, scales = mla.new_pool(d, inp.num_pages, DEV)
    if poison:
        poison_pool(pool, scales)
    mla.append_latent(d, t["c_kv"], t["k_pe"], t["positions"], t["seq_ids"], t["block_table"],
                      pool, scales, rope=rope)
    return pool, scales, t


def decode_step(inp, d, num_splits=0, dev_inputs=None, cache=None):
    """append (all tokens) -> absorb -> decode -> out_proj; returns host numpy results."""
    if cache is None:
        pool, scales, t = build_cache(inp, d, dev_inputs)
    else:
        pool, scales, t = cache
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    o_lat, lse = mla.decode_paged(d, q, pool, scales, t["block_table"], t["seq_lens"],
                                  num_splits=num_splits)
    out = mla.out_proj(d, o_lat, t["w_uv"])
    torch.cuda.synchronize()
    return {
        "q": q.float().cpu().numpy().astype(np.float64),
        "o_lat": o_lat.float().cpu().numpy().astype(np.float64),
        "lse": lse.cpu().numpy().astype(np.float64),
        "out": out.float().cpu().numpy().astype(np.float64),
        "o_lat_dev": o_lat, "lse_dev": lse, "pool": pool, "scales": scales, "t": t,
    }


def rel_l2(x, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def max_abs(x, ref):
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


# Tolerance for bf16 inputs with fp32 accumulation, over the whole compared
# tensor: max |gpu - ref| <= 2e-2 and ||gpu - ref|| / ||ref|| <= 5e-3.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def assert_close(x, ref, what, max_abs_tol=MAX_ABS, rel_tol=REL_L2):
    """Checks the bar and prints the achieved margin (`[margin]` lines, shown
    with pytest -s, are the source of the per-workload margin table)."""
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    ma, rl = max_abs(x, ref), rel_l2(x, ref)
    print(f"[margin] {what}: max_abs={ma:.3e} rel_l2={rl:.3e} (bar {max_abs_tol:g} / {rel_tol:g})",
          flush=True)
    assert ma <= max_abs_tol and rl <= rel_tol, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl


def unused_mask(inp):
    spare, tail = unused_slots(inp)
    return spare, tail
