"""The library keeps no per-call state: calls from two host threads at once,
each on its own stream with its own workspace and outputs, must reproduce the
single-threaded results bit for bit (decode and decode with the merged
projection, at different split counts).  ctypes releases the GIL around each
foreign call, so the host side of the calls really overlaps."""
import threading

import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from workload import configs, make_inputs
from workload.torch_io import bf16_bits

from gpu_util import DEV, build_cache, dims_for

pytestmark = pytest.mark.gpu

ITERS = 25


def test_two_threads_two_streams_match_single_thread():
    wl = configs.V3.with_(name="v3_threads", batch=5, seq_len=None, seq_lens=(1, 31, 33, 1500, 64))
    print("[threads] two host threads, two streams, decode and decode_out", flush=True)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    q = mla.absorb_q(d, t["q_nope"], t["q_pe"], t["q_pos"], t["w_uk"])
    args = (d, q, pool, scales, t["block_table"], t["seq_lens"])
    splits = (0, 3)
    ref = {}
    for ns in splits:
        o, l = mla.decode_paged(*args, num_splits=ns)
        out, _, _ = mla.decode_paged_out(*args, t["w_uv"], num_splits=ns)
        ref[ns] = (bf16_bits(o), l.cpu().numpy(), bf16_bits(out))
    torch.cuda.synchronize()

    errors = []

    def worker(ns):
        try:
            s = torch.cuda.Stream()
            got = []
            with torch.cuda.stream(s):
                ws = mla.new_workspace(d, wl.batch, ns, DEV)
                for _ in range(ITERS):
                    o, l = mla.decode_paged(*args, num_splits=ns, workspace=ws)
                    out, _, _ = mla.decode_paged_out(*args, t["w_uv"], num_splits=ns, workspace=ws)
                    got.append((o, l, out))
            s.synchronize()
            for o, l, out in got:
                assert np.array_equal(bf16_bits(o), ref[ns][0]), f"o_lat, splits {ns}"
                assert np.array_equal(l.cpu().numpy(), ref[ns][1]), f"lse, splits {ns}"
                assert np.array_equal(bf16_bits(out), ref[ns][2]), f"out, splits {ns}"
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(ns,)) for ns in splits]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
