"""The decode step (append -> absorb -> decode -> out-projection, or with the
out-projection in the decode call's merge kernel) captured in a
HIP graph and replayed: the library only enqueues kernels on the caller's
stream (no allocation, no host synchronisation, no memset), so the step can be
captured as is.  Every replay, with eager work and synchronisations between
replays, must give the eager step's outputs bit for bit (the kernels are
deterministic), also after the inputs are rewritten in place between replays.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from workload import configs, make_inputs
from workload.torch_io import to_device

from gpu_util import DEV, dims_for, poison_pool

pytestmark = pytest.mark.gpu

CASES = [
    configs.V3.with_(name="v3_graph", batch=6, seq_len=None, seq_lens=(1, 40, 700, 64, 2000, 33)),
    configs.V2LITE.with_(name="v2lite_graph", batch=4, seq_len=None, seq_lens=(100, 1, 900, 64)),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate_calls", "append_absorb+decode_out"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_captured_step_replays_bit_for_bit(wl, fused):
    inp = make_inputs(wl)
    d = dims_for(wl)
    t = to_device(inp, DEV)
    B, H, R = wl.batch, wl.n_heads, wl.d_latent
    pool, scales = mla.new_pool(d, inp.num_pages, DEV)
    poison_pool(pool, scales)
    # the cache holds every token but the last of each sequence; the step
    # appends the last one
    last = (inp.cu_seqlens[1:] - 1).astype(np.int64)
    keep = np.ones(inp.total_tokens, bool)
    keep[last] = False
    ik, il = torch.from_numpy(np.nonzero(keep)[0]).to(DEV), torch.from_numpy(last).to(DEV)
    mla.append_latent(d, t["c_kv"][ik].contiguous(), t["k_pe"][ik].contiguous(),
                      t["positions"][ik].contiguous(), t["seq_ids"][ik].contiguous(),
                      t["block_table"], pool, scales)
    new = {k: t[k][il].contiguous() for k in ("c_kv", "k_pe", "positions", "seq_ids")}
    ws = mla.new_workspace(d, B, 0, DEV)
    q = torch.empty((B, H, R), dtype=torch.bfloat16, device=DEV)
    o_lat = torch.empty((B, H, wl.d_c), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    out = torch.empty((B, H, wl.d_v), dtype=torch.bfloat16, device=DEV)
    q_nope = t["q_nope"].clone()

    def step():
        if fused:
            mla.append_absorb(d, new["c_kv"], new["k_pe"], new["positions"], new["seq_ids"],
                              t["block_table"], pool, scales, q_nope, t["q_pe"], t["q_pos"], t["w_uk"], q)
        else:
            mla.append_latent(d, new["c_kv"], new["k_pe"], new["positions"], new["seq_ids"],
                              t["block_table"], pool, scales)
            mla.absorb_q(d, q_nope, t["q_pe"], t["q_pos"], t["w_uk"], q)
        if fused:
            mla.decode_paged_out(d, q, pool, scales, t["block_table"], t["seq_lens"], t["w_uv"], 0, ws,
                                 out, o_lat, lse)
        else:
            mla.decode_paged(d, q, pool, scales, t["block_table"], t["seq_lens"], 0, ws, o_lat, lse)
            mla.out_proj(d, o_lat, t["w_uv"], out)

    def snapshot():
        return [x.clone() for x in (q, o_lat, lse, out)]

    step()
    torch.cuda.synchronize()
    eager = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    def same(a, b):
        return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
                   for x, y in zip(a, b))

    for i in range(4):
        for x in (q, o_lat, lse, out):           # eager work between replays
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(snapshot(), eager), f"replay {i} differs from the eager step"

    # new query values written in place: the replay reads them
    q_nope.copy_(torch.flip(t["q_nope"], dims=[0]))
    step()
    torch.cuda.synchronize()
    eager2 = snapshot()
    assert not same(eager2, eager)
    for i in range(2):
        for x in (q, o_lat, lse, out):
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(snapshot(), eager2), f"replay {i} after the input update differs"


def test_captured_prefill_replays_bit_for_bit():
    """mla_prefill_paged (both up-projections and the attention) captured and
    replayed, with eager work between replays: bit for bit the eager call."""
    wl = configs.V3.with_(name="v3_prefill_graph", batch=2, n_heads=8, seq_len=None,
                          seq_lens=(300, 700), q_len=200)
    inp = make_inputs(wl)
    d = dims_for(wl)
    t = to_device(inp, DEV)
    B, ql, H = wl.batch, wl.q_len, wl.n_heads
    pool, scales = mla.new_pool(d, inp.num_pages, DEV)
    mla.append_latent(d, t["c_kv"], t["k_pe"], t["positions"], t["seq_ids"], t["block_table"],
                      pool, scales)
    qn = t["q_nope"].reshape(B * ql, H, wl.d_nope).contiguous()
    qp = t["q_pe"].reshape(B * ql, H, wl.d_rope).contiguous()
    q_start = torch.tensor([0, ql, 2 * ql], dtype=torch.int32, device=DEV)
    ws = torch.empty(mla.prefill_workspace_size(d, B, inp.max_pages), dtype=torch.uint8, device=DEV)
    out = torch.empty((B * ql, H, wl.d_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B * ql, H), dtype=torch.float32, device=DEV)

    def call():
        mla.prefill_paged(d, qn, qp, q_start, ql, pool, scales, t["block_table"], t["seq_lens"],
                          t["w_uk"], t["w_uv"], ws, out, lse)

    call()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        lse.zero_()
        ws.zero_()                               # the workspace is rebuilt by every call
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16)), f"replay {i}: out"
        assert torch.equal(lse, eager[1]), f"replay {i}: lse"
