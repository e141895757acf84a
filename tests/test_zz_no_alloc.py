"""mla_decode_paged_noalloc (workspace in the library's device array) against
mla_decode_paged / mla_decode_paged_multi with a caller workspace, on the same
inputs: three calls in a row, each smaller than the one before, so every call
runs on the array as the previous one left it.  The outputs must equal the
workspace call's bit for bit (same kernels, same split), and meet the oracle
bar."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import reference_decode, reference_decode_multi
from workload import configs, make_inputs

from gpu_util import assert_close, build_cache, dims_for

pytestmark = pytest.mark.gpu

CASES = [
    configs.V3.with_(name="noalloc_v3", batch=6, seq_len=None, seq_lens=(1, 700, 2048, 33, 4000, 129)),
    configs.V3.with_(name="noalloc_v3_fp8", fp8=True, batch=3, seq_len=None, seq_lens=(300, 1000, 64)),
    configs.V2LITE.with_(name="noalloc_v2lite_q2", batch=3, seq_len=None, seq_lens=(5, 300, 64), q_len=2),
]


def test_noalloc_matches_workspace_calls():
    for wl in CASES:
        print(f"[noalloc] {wl.name}", flush=True)
        inp = make_inputs(wl)
        d = dims_for(wl)
        pool, scales, t = build_cache(inp, d)
        B, ql, H, R = wl.batch, wl.q_len, wl.n_heads, wl.d_c + wl.d_rope
        q = mla.absorb_q(d, t["q_nope"].reshape(B * ql, H, wl.d_nope), t["q_pe"].reshape(B * ql, H, wl.d_rope),
                         t["q_pos"].reshape(B * ql).contiguous(), t["w_uk"])
        if ql == 1:
            o_ws, l_ws = mla.decode_paged(d, q, pool, scales, t["block_table"], t["seq_lens"])
            o_na, l_na = mla.decode_paged_noalloc(d, q, pool, scales, t["block_table"], t["seq_lens"])
        else:
            q4 = q.view(B, ql, H, R)
            o_ws, l_ws = mla.decode_paged_multi(d, q4, pool, scales, t["block_table"], t["seq_lens"])
            o_na, l_na = mla.decode_paged_noalloc(d, q4, pool, scales, t["block_table"], t["seq_lens"])
        torch.cuda.synchronize()
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), wl.name
        assert torch.equal(l_na, l_ws), wl.name
        ref = reference_decode(inp) if ql == 1 else reference_decode_multi(inp)
        got = o_na.float().cpu().numpy().astype(np.float64)
        assert_close(got, ref["o_lat"], f"{wl.name} o_lat (no-alloc)")
        assert np.max(np.abs(l_na.cpu().numpy() - ref["lse"])) <= 1e-2
