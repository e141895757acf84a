"""mla_absorb_q and mla_out_proj on the GPU against the oracle's absorbed-form
steps (fp64), on the tiny, V2-Lite and V3 head shapes."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import absorb_query, bf16_bits_to_f64, out_projection, rope
from workload import configs, f32_to_bf16_bits, make_inputs
from workload.torch_io import bf16_bits, bf16_tensor, to_device

from gpu_util import DEV, assert_close, dims_for

pytestmark = pytest.mark.gpu

SHAPES = [configs.TINY,
          configs.V2LITE.with_(seq_len=64),
          configs.V3.with_(seq_len=32),
          configs.V3.with_(batch=37, seq_len=32),       # ragged batch tail (not a multiple of 32)
          configs.V3.with_(batch=1, n_heads=20, seq_len=32)]


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: f"{w.name}_B{w.batch}_H{w.n_heads}")
def test_absorb_q(wl):
    inp = make_inputs(wl)
    d = dims_for(wl)
    t = to_device(inp, DEV)
    print(f"[absorb] {wl.name} B={wl.batch} H={wl.n_heads}", flush=True)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(bf16_bits(q))
    ref = absorb_query(bf16_bits_to_f64(inp.q_nope), bf16_bits_to_f64(inp.q_pe),
                       bf16_bits_to_f64(inp.w_uk), inp.q_pos(), wl.rope_base)
    assert_close(got[..., :wl.d_c], ref[..., :wl.d_c], "q_lat")
    # the rotated part is one rounding (fp64 -> fp32 -> bf16) away from the
    # oracle: at most 1e-3 of the values differ from that rounding (an fp32
    # result that lands across a bf16 midpoint), and every value is within one
    # bf16 step (2^-8 relative) of the fp64 rotation
    kr = ref[..., wl.d_c:]
    want = f32_to_bf16_bits(kr.astype(np.float32))
    got_rot = bf16_bits(q)[..., wl.d_c:]
    assert np.mean(got_rot != want) <= 1e-3
    err = np.abs(bf16_bits_to_f64(got_rot) - kr)
    assert np.all(err <= 2.0 ** -8 * np.abs(kr) + 1e-30), float(np.max(err / (np.abs(kr) + 1e-30)))


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: f"{w.name}_B{w.batch}_H{w.n_heads}")
def test_out_proj(wl):
    inp = make_inputs(wl)
    d = dims_for(wl)
    rng = np.random.default_rng(1)
    o_bits = f32_to_bf16_bits(rng.standard_normal((wl.batch, wl.n_heads, wl.d_c)).astype(np.float32) * 0.05)
    print(f"[out_proj] {wl.name} B={wl.batch} H={wl.n_heads}", flush=True)
    out = mla.out_proj(d, bf16_tensor(o_bits, DEV), bf16_tensor(inp.w_uv, DEV))
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(bf16_bits(out))
    ref = out_projection(bf16_bits_to_f64(o_bits), bf16_bits_to_f64(inp.w_uv))
    assert_close(got, ref, "out", max_abs_tol=2e-3)
