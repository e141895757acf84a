"""The timed entry points (mla_decode_paged_timed, mla_prefill_paged_timed and
the event arguments of mla_decode_paged_out) on the GPU: the caller's events
only bracket the attention kernel, so every output must be bit-identical to
the untimed call on the same inputs, and the events must have been recorded
around real work (elapsed time positive and below the whole call's)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from workload import configs, make_inputs
from workload.torch_io import bf16_bits

from gpu_util import DEV, build_cache, dims_for
from test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _check_elapsed(ev, what):
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    print(f"[timed] {what}: {1000 * ms:.1f} us between the events", flush=True)
    assert 0.0 < ms < 1000.0, ms


def _same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    if a.dtype == torch.bfloat16:
        assert np.array_equal(bf16_bits(a), bf16_bits(b)), what
    else:
        assert torch.equal(a, b), what


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_decode_timed_matches_untimed(fp8, num_splits):
    wl = configs.V3.with_(name="v3_timed", fp8=fp8, batch=5, seq_len=None, seq_lens=(1, 31, 33, 1500, 64))
    print(f"[timed decode] fp8={fp8} splits={num_splits}", flush=True)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    args = (d, q, pool, scales, t["block_table"], t["seq_lens"])
    o0, l0 = mla.decode_paged(*args, num_splits=num_splits)
    ev = _events()
    o1, l1 = mla.decode_paged(*args, num_splits=num_splits, events=ev)
    _check_elapsed(ev, "decode_paged")
    _same(o0, o1, "o_lat")
    _same(l0, l1, "lse")
    # with the projection merged in: out, o_lat and lse
    r0 = mla.decode_paged_out(*args, t["w_uv"], num_splits=num_splits, want_o_lat=True, want_lse=True)
    ev = _events()
    r1 = mla.decode_paged_out(*args, t["w_uv"], num_splits=num_splits, want_o_lat=True, want_lse=True,
                              events=ev)
    _check_elapsed(ev, "decode_paged_out")
    for a, b, what in zip(r0, r1, ("out", "o_lat", "lse")):
        _same(a, b, what)


def test_decode_multi_timed_matches_untimed():
    wl = configs.V3.with_(name="v3_q2_timed", batch=3, seq_len=None, seq_lens=(2, 65, 1500), q_len=2)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    B, ql, H = wl.batch, wl.q_len, wl.n_heads
    q = mla.absorb_q(d, t["q_nope"].reshape(B * ql, H, wl.d_nope), t["q_pe"].reshape(B * ql, H, wl.d_rope),
                     t["q_pos"].reshape(B * ql).contiguous(), t["w_uk"]).view(B, ql, H, wl.d_latent)
    args = (d, q, pool, scales, t["block_table"], t["seq_lens"])
    o0, l0 = mla.decode_paged_multi(*args)
    ev = _events()
    o1, l1 = mla.decode_paged_multi(*args, events=ev)
    _check_elapsed(ev, "decode_paged_multi")
    _same(o0, o1, "o_lat")
    _same(l0, l1, "lse")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_prefill_timed_matches_untimed(fp8):
    wl = configs.V3.with_(name="v3_pf_timed", fp8=fp8, batch=2, n_heads=4, seq_len=None, seq_lens=(700, 300),
                          q_len=150)
    inp = make_inputs(wl)
    d = dims_for(wl)
    cache = build_cache(inp, d)
    out0, lse0, _, _ = run_prefill(inp, d, cache=cache)
    ev = _events()
    out1, lse1, _, _ = run_prefill(inp, d, cache=cache, events=ev)
    _check_elapsed(ev, "prefill_paged")
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1, equal_nan=True)
