"""mla_append_absorb (the step's append and query absorption in one launch)
against the two separate calls on the same inputs: pool bytes, fp8 scales and
the absorbed queries bit for bit, bf16 and fp8 caches, both supported widths,
and no new tokens (absorption only)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from workload import configs, make_inputs
from workload.torch_io import to_device

from gpu_util import DEV, dims_for, poison_pool

pytestmark = pytest.mark.gpu

CASES = [
    configs.TINY,
    configs.V3.with_(name="v3_aa", batch=6, seq_len=None, seq_lens=(1, 40, 700, 64, 2000, 33)),
    configs.V3.with_(name="v3_aa_fp8", fp8=True, batch=5, seq_len=None, seq_lens=(5, 99, 300, 64, 1)),
    configs.V2LITE.with_(name="v2lite_aa_b70", batch=70, seq_len=None,
                         seq_lens=tuple(int(x) for x in np.arange(70) % 37 + 1)),
]


def _bytes(t):
    return t.view(torch.uint8).cpu().numpy() if t is not None else None


@pytest.mark.parametrize("new_tokens", [True, False], ids=["append", "no_tokens"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_append_absorb_equals_the_two_calls(wl, new_tokens):
    inp = make_inputs(wl)
    d = dims_for(wl)
    t = to_device(inp, DEV)
    print(f"[append_absorb] {wl.name} new_tokens={new_tokens}", flush=True)
    n = inp.total_tokens if new_tokens else 0
    sel = slice(0, n)
    results = []
    for fused in (False, True):
        pool, scales = mla.new_pool(d, inp.num_pages, DEV)
        poison_pool(pool, scales)
        q = torch.full((wl.batch, wl.n_heads, wl.d_latent), 7.0, dtype=torch.bfloat16, device=DEV)
        args = (t["c_kv"][sel].contiguous(), t["k_pe"][sel].contiguous(), t["positions"][sel].contiguous(),
                t["seq_ids"][sel].contiguous(), t["block_table"], pool, scales)
        if fused:
            mla.append_absorb(d, *args, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"], q)
        else:
            mla.append_latent(d, *args)
            mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"], q)
        torch.cuda.synchronize()
        results.append((_bytes(pool), _bytes(scales), _bytes(q)))
    (p0, s0, q0), (p1, s1, q1) = results
    assert np.array_equal(p0, p1)
    assert (s0 is None and s1 is None) or np.array_equal(s0, s1)
    assert np.array_equal(q0, q1)
    assert not np.any(q1.view(np.uint16) == 0x40E0)            # every q element written (7.0 poison gone)
