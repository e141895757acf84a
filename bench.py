#!/usr/bin/env python3
"""Benchmark of one MLA absorbed-decode step on one MI355X.

A step is the whole hot path for one new token per sequence:
  mla_append_absorb (mla_append_latent of the B new rows and mla_absorb_q in
  one launch) -> mla_decode_paged_out
  (split attention with its own tile plan, then the LSE merge and the W_UV
  output projection in one kernel),
on the DeepSeek-V3-shaped workload (B=64, H=128, d_c=512, d_rope=64,
d_nope=d_v=128, S=8192, page 64, bf16 latent cache, permuted pages), with all
inputs resident in HBM.  The cache holds S-1 tokens per sequence before the
timed region; every step appends token S-1 (the same slot each step) and
attends over all S tokens.

`--workload v3mtp2` runs the same step for two new tokens per sequence scored
in one pass (the q_len form of the same call; the verification of
multi-token-prediction drafts); its tokens/s counts the B * q_len scored tokens.

Prints one JSON line: whole-step decode tokens/s, plus
  roofline: the split-attention kernel's achieved HBM bandwidth
            (algorithmic bytes per launch / its mean duration, HIP events on
            the launch stream) against 8 TB/s,
  cpu_baseline: the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + achieved TB/s & % roofline, B=64 S=8192 H=128"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3", choices=["v3", "v2lite", "ragged", "fp8long", "v3mtp2"])
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=24,
                    help="sequences of the workload the oracle decodes for cpu_baseline (0 = skip)")
    ap.add_argument("--flushed-iters", type=int, default=50,
                    help="decode-only iterations, each after reading 768 MiB of other data "
                         "(evicts the Infinity Cache), for the median / p10 / p90 (0 = skip)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as a captured HIP graph (replays) instead of eager calls; "
                         "the eager pass still runs for the split kernel's timing")
    ap.add_argument("--op", default="step", choices=["step", "project_append", "prefill"],
                    help="step: the decode step (default); project_append: mla_project_append "
                         "alone for one decode step's new tokens (B=64, d_model=7168, V3 rows); "
                         "prefill: mla_prefill_paged on a 4096-token chunk of two 8192-token "
                         "sequences (V3 heads)")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="only time the fp64 oracle on a bounded sample of every workload (host "
                         "cores, no GPU) and print one JSON line per workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run three device-to-device copies of MIB MiB (a kernel of known "
                         "traffic, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's main kernel (k_split, or
    k_prefill for v3prefill) from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the kernel sources changed since it was taken or
    the workload differs."""
    import hashlib
    import re
    name = {"v3": "k_split_v3_b64_s8192.md", "v3mtp2": "k_split_v3mtp2_b64_q2_s8192.md",
            "v2lite": "k_split_v2lite_b16_s4096.md", "ragged": "k_split_ragged_b128_s512-32768.md",
            "fp8long": "k_split_fp8long_b4_s131072.md",
            "v3prefill": "k_prefill_v3_b2_s8192_c4096.md"}.get(workload)
    if name is None:
        return None
    path = os.path.join(ROOT, "profiles", name)
    try:
        text = open(path, encoding="utf-8").read()
        block = json.loads(re.search(r"```json\n(.*?)```", text, re.S).group(1))
    except (OSError, AttributeError, ValueError):
        return None
    if block.get("workload") != workload:
        return None
    for rel, digest in block["sources_sha256"].items():
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return int(block["traffic_bytes_per_launch"])


def bench_project_append(args):
    """mla_project_append for the 64 new tokens of a V3 decode step: hidden
    states [64][7168] projected by w_down [576][7168] and appended at position
    8191 of 64 sequences (permuted pages).  The roof is HBM: the weight, the
    hidden states and the rows written, each moved once."""
    import numpy as np
    import torch

    import mla_latent_kv_nope_amd as mla
    from workload import configs, make_projection_inputs
    from workload.torch_io import bf16_tensor

    wl, d_model = configs.V3, 7168
    B, S, R = wl.batch, wl.seq_len, wl.d_latent
    dev = "cuda:0"
    torch.cuda.set_device(0)
    d = mla.make_dims(wl.n_heads, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v, wl.page_size,
                      softmax_scale=wl.softmax_scale, rope_base=wl.rope_base)
    pin = make_projection_inputs(B, d_model, R, seed=0)
    h, w = bf16_tensor(pin.h, dev), bf16_tensor(pin.w_down, dev)
    mp = S // wl.page_size
    rng = np.random.default_rng(0)
    bt = torch.from_numpy(rng.permutation(B * mp).astype(np.int32).reshape(B, mp)).to(dev)
    pool, _ = mla.new_pool(d, B * mp, dev)
    pos = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
    sid = torch.arange(B, dtype=torch.int32, device=dev)
    ws = torch.empty(mla.project_append_workspace_size(d, d_model, B), dtype=torch.uint8, device=dev)
    call = lambda: mla.project_append(d, h, w, pos, sid, bt, pool, None, ws)
    settled = settle(torch, call)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    nbytes = R * d_model * 2 + B * d_model * 2 + B * R * 2
    flops = 2.0 * B * R * d_model
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "mla_project_append time per decode step (64 new tokens)", "value": round(us, 3),
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle": settled,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "V3 decode step's new tokens: T=64, d_model=7168 -> 576-wide rows, "
                               "page 64, permuted pages", "tokens": B, "d_model": d_model,
                   "kernels": "k_down (split-K, 18 x 28 workgroups) + k_append (chunk sum)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_call": nbytes, "flops_per_call": flops,
                     "note": "both kernels of the call, back to back; HIP events on the stream"},
    }), flush=True)


def bench_prefill(args):
    """mla_prefill_paged on the second 4096-token chunk of two 8192-token
    sequences (DeepSeek-V3 heads: H=128, latent 512, RoPE 64, K/V width 128;
    page 64, permuted pages): the up-projection of all 8192 cached rows per
    sequence to K_nope and V, then causal attention of the 4096 new tokens.
    The roof is the bf16 MFMA rate: the attention kernel's algorithmic FLOPs
    (each new token against the keys at positions <= its own) per launch over
    its duration (HIP events on the launch stream)."""
    import torch

    import mla_latent_kv_nope_amd as mla
    from workload import configs, make_inputs
    from workload.torch_io import to_device

    wl = configs.V3.with_(name="v3prefill", batch=2, seq_len=8192, q_len=4096)
    B, S, n, H = wl.batch, wl.seq_len, wl.q_len, wl.n_heads
    dev = "cuda:0"
    torch.cuda.set_device(0)
    d = mla.make_dims(H, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v, wl.page_size,
                      softmax_scale=wl.softmax_scale, rope_base=wl.rope_base)
    inp = make_inputs(wl)
    t = to_device(inp, dev)
    pool, _ = mla.new_pool(d, inp.num_pages, dev)
    mla.append_latent(d, t["c_kv"], t["k_pe"], t["positions"], t["seq_ids"], t["block_table"], pool, None)
    qn = t["q_nope"].reshape(B * n, H, wl.d_nope).contiguous()
    qp = t["q_pe"].reshape(B * n, H, wl.d_rope).contiguous()
    q_start = torch.tensor([0, n, 2 * n], dtype=torch.int32, device=dev)
    ws = torch.empty(mla.prefill_workspace_size(d, B, inp.max_pages), dtype=torch.uint8, device=dev)
    out = torch.empty((B * n, H, wl.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B * n, H), dtype=torch.float32, device=dev)
    call = lambda ev=None: mla.prefill_paged(d, qn, qp, q_start, n, pool, None, t["block_table"],
                                             t["seq_lens"], t["w_uk"], t["w_uv"], ws, out, lse, events=ev)
    settled = settle(torch, call)
    for _ in range(args.warmup):
        call()
    evs = kernel_events(torch, args.steps)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        call(evs[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    attn_us = mean_event_ms(evs) * 1e3
    # new token i sits at position S - n + i and sees S - n + i + 1 keys
    keys = n * (S - n) + n * (n + 1) // 2
    attn_flops = 2.0 * B * H * keys * (wl.d_nope + wl.d_rope + wl.d_v)
    up_flops = 2.0 * B * S * wl.d_c * (wl.d_nope + wl.d_v) * H
    tflops = attn_flops / (attn_us * 1e-6) / 1e12
    line = {
        "metric": "MLA explicit-form prefill tokens/s (chunk of 4096 new tokens on 8192-token "
                  "sequences, H=128)",
        "value": round(B * n / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "V3 prefill chunk: B=2, S=8192, 4096 new tokens each (the second "
                               "chunk), H=128, d_c=512, d_rope=64, d_nope=d_v=128, page 64, "
                               "permuted pages",
                   "kernels": "k_up (K_nope and V^T of all cached rows) + k_prefill (causal attention)",
                   "up_projection_us": round(ms * 1e3 - attn_us, 2), "attention_us": round(attn_us, 2),
                   "attention_flops": attn_flops, "up_projection_flops": up_flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("v3prefill"), "kernel": "k_prefill",
                     "note": "algorithmic FLOPs of the attention per launch / its mean duration "
                             "(HIP events on the launch stream)"},
    }
    if args.cpu_sample > 0:
        line["cpu_baseline"] = cpu_baseline_prefill(inp)
    print(json.dumps(line), flush=True)


# GPU time the step runs untimed before the counted warm-up steps.  From idle
# the GPU needs tens of milliseconds of load to reach its steady clocks:
# measured, 20 timed V3 steps after 5 warm-up steps took 176 us per split
# launch, after 200 warm-up steps (about 38 ms) 152 us.
SETTLE_MS = 100.0


def settle(torch, fn, min_ms: float = SETTLE_MS) -> dict:
    """Runs fn() untimed until at least min_ms of wall time have passed (the
    GPU kept busy: a synchronise every 20 calls), then synchronises."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            break
    return {"calls": n, "ms": round((time.perf_counter() - t0) * 1e3, 1),
            "why": "untimed, before the warm-up steps: the GPU leaves its idle clock state"}


def kernel_events(torch, n: int):
    """n (start, stop) event pairs for the library's timed entry points, each
    event created (by one record) before the timed region starts."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        b.record()
    return evs


def mean_event_ms(evs) -> float:
    """Mean milliseconds between the events of each pair (after a synchronise)."""
    return sum(a.elapsed_time(b) for a, b in evs) / max(1, len(evs))


def cpu_baseline_prefill(inp):
    """The oracle's explicit-form prefill on a bounded sample: sequence 0,
    every second head (64 of 128), all 4096 new tokens.  Scaled to tokens/s
    of the whole workload as (rows * heads / H) / time."""
    from oracle import reference_prefill
    wl = inp.wl
    heads = list(range(0, wl.n_heads, 2))
    rows = list(range(wl.q_len))
    t0 = time.perf_counter()
    reference_prefill(inp, batches=[0], heads=heads, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(len(rows) * len(heads) / wl.n_heads / dt, 3), "unit": "tokens/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"sequence 0, {len(heads)} of {wl.n_heads} heads (every second), all "
                      f"{len(rows)} new tokens, {dt:.1f} s"}


def cpu_baseline(inp, n_seq: int):
    """Time the oracle (explicit fp64 form) on the first n_seq sequences."""
    import numpy as np
    from oracle import reference_decode, reference_decode_multi
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    ql = inp.wl.q_len
    t0 = time.perf_counter()
    if ql == 1:
        reference_decode(inp, batches=range(n_seq))
    else:
        reference_decode_multi(inp, batches=range(n_seq))
    dt = time.perf_counter() - t0
    toks = int(np.sum(inp.seq_lens[:n_seq]))
    return {"value": n_seq * ql / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_seq} of {len(inp.seq_lens)} sequences x {ql} new token(s) x "
                      f"{inp.wl.n_heads} heads ({toks} cached tokens), explicit fp64 form, {dt:.2f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
            "blas": _blas_name()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_name() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} ({p.get('num_threads')} threads)" for p in threadpool_info()
                if p.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:  # pragma: no cover
        return "unknown"


def flushed_decode_times(mla, torch, decode, iters: int):
    """Per-call time of mla_decode_paged alone (HIP events on the current
    stream), each call right after a full read of a 768 MiB scratch buffer, so
    that no line of the previous call survives in the 256 MB Infinity Cache.
    (A read keeps the GPU busy up to the call: after idle gaps or large
    writes the clock state alone moved this time by up to 30 %.)"""
    scratch = torch.ones(768 << 18, dtype=torch.int32, device="cuda:0")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for _ in range(3):
        decode()
    for e0, e1 in ev:
        scratch.max()
        e0.record()
        decode()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    pick = lambda f: ms[min(len(ms) - 1, int(f * len(ms)))]
    return {"median_ms": round(pick(0.5), 5), "p10_ms": round(pick(0.1), 5),
            "p90_ms": round(pick(0.9), 5), "iters": iters,
            "note": "split + combine, each call after reading 768 MiB of other data"}


# sequences of each workload the oracle decodes for --cpu-baseline-all (about
# 5-15 s of host time each)
CPU_SAMPLE_ALL = {"v2lite": 16, "v3": 24, "ragged": 16, "fp8long": 1, "v3mtp2": 12}


def cpu_baseline_all():
    """The oracle as it stands, timed on every workload's bounded sample in one
    run (the default bench line carries only its own workload's)."""
    from workload import configs, make_inputs
    for name, n_seq in CPU_SAMPLE_ALL.items():
        inp = make_inputs(configs.get(name))
        # a sample under 5 s (the whole small workload) is repeated and averaged
        runs, spent = [], 0.0
        while spent < 5.0:
            t0 = time.perf_counter()
            runs.append(cpu_baseline(inp, n_seq))
            spent += time.perf_counter() - t0
        base = dict(runs[-1])
        base["value"] = sum(r["value"] for r in runs) / len(runs)
        if len(runs) > 1:
            base["sample"] += f"; mean of {len(runs)} runs"
        rec = {"workload": name, "description": inp.wl.description, "cpu_baseline": base}
        print(json.dumps(rec), flush=True)
        del inp
    from workload import configs as c
    wl = c.V3.with_(name="v3prefill", batch=2, seq_len=8192, q_len=4096)
    inp = make_inputs(wl)
    print(json.dumps({"workload": "v3prefill", "description": "prefill chunk of 4096 new tokens in "
                      "two 8192-token sequences, H=128", "cpu_baseline": cpu_baseline_prefill(inp)}),
          flush=True)


def main():
    args = parse()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.cpu_baseline_all:
        cpu_baseline_all()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures exactly one GPU; the decode path shards by sequence "
              "(attention data parallel) and needs no collective, but multi-GPU runs are not "
              "part of it. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.op == "project_append":
        bench_project_append(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return

    import numpy as np
    import torch

    import mla_latent_kv_nope_amd as mla
    from workload import configs, make_inputs
    from workload.torch_io import to_device

    wl = configs.get(args.workload)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = make_inputs(wl)
    d = mla.make_dims(wl.n_heads, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v, wl.page_size, fp8=wl.fp8,
                      softmax_scale=wl.softmax_scale, rope_base=wl.rope_base)
    t = to_device(inp, dev)
    B, H = wl.batch, wl.n_heads
    R = wl.d_c + wl.d_rope
    ql = wl.q_len
    BQ = B * ql                       # query rows per step

    # cache: every token but the last q_len of each sequence
    cu = inp.cu_seqlens
    last = (cu[1:, None] - ql + np.arange(ql)[None, :]).reshape(-1).astype(np.int64)
    keep = np.ones(inp.total_tokens, bool)
    keep[last] = False
    idx_keep = torch.from_numpy(np.nonzero(keep)[0]).to(dev)
    idx_last = torch.from_numpy(last).to(dev)
    pool, scales = mla.new_pool(d, inp.num_pages, dev)
    mla.append_latent(d, t["c_kv"][idx_keep].contiguous(), t["k_pe"][idx_keep].contiguous(),
                      t["positions"][idx_keep].contiguous(), t["seq_ids"][idx_keep].contiguous(),
                      t["block_table"], pool, scales)
    new_c = t["c_kv"][idx_last].contiguous()
    new_k = t["k_pe"][idx_last].contiguous()
    new_pos = t["positions"][idx_last].contiguous()
    new_sid = t["seq_ids"][idx_last].contiguous()
    del t["c_kv"], t["k_pe"]

    ws = mla.new_workspace(d, BQ, args.num_splits, dev)
    q = torch.empty((BQ, H, R), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty((BQ, H, wl.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((BQ, H), dtype=torch.float32, device=dev)
    out = torch.empty((BQ, H, wl.d_v), dtype=torch.bfloat16, device=dev)
    q_nope = t["q_nope"].reshape(BQ, H, wl.d_nope)
    q_pe = t["q_pe"].reshape(BQ, H, wl.d_rope)
    q_pos = t["q_pos"].reshape(BQ).contiguous()

    # ev: (start, stop) events recorded around the split kernel on the stream
    if ql == 1:
        def decode(ev=None):
            mla.decode_paged(d, q, pool, scales, t["block_table"], t["seq_lens"], args.num_splits,
                             ws, o_lat, lse, events=ev)
    else:
        def decode(ev=None):
            mla.decode_paged_multi(d, q.view(B, ql, H, R), pool, scales, t["block_table"],
                                   t["seq_lens"], args.num_splits, ws, o_lat.view(B, ql, H, wl.d_c),
                                   lse.view(B, ql, H), events=ev)

    # the step: the append and the query absorption in one launch, then decode
    # with the W_UV projection in its merge kernel (o_lat and lse are not
    # needed downstream and are not written)
    def step(ev=None):
        mla.append_absorb(d, new_c, new_k, new_pos, new_sid, t["block_table"], pool, scales,
                          q_nope, q_pe, q_pos, t["w_uk"], q)
        mla.decode_paged_out(d, q.view(B, ql, H, R), pool, scales, t["block_table"], t["seq_lens"],
                             t["w_uv"], args.num_splits, ws, out.view(B, ql, H, wl.d_v), events=ev)

    settled = settle(torch, step)
    for _ in range(args.warmup):
        step()
    evs = kernel_events(torch, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    split_ms = mean_event_ms(evs)
    n_rec = len(evs)
    assert torch.isfinite(out.float()).all(), "non-finite output"
    eager_elapsed = elapsed
    if args.graph:
        # capture the step (warm-up on the capture stream first), then time replays
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert torch.isfinite(out.float()).all(), "non-finite output (graph)"
    flushed = None
    if args.flushed_iters > 0:
        flushed = flushed_decode_times(mla, torch, decode, args.flushed_iters)

    ms_step = 1e3 * elapsed / args.steps
    value = BQ * args.steps / elapsed
    total_tokens = int(inp.total_tokens)
    bpt = mla.cache_bytes_per_token(d)
    # cache rows (each read once) + the absorbed query rows
    split_bytes = total_tokens * bpt + BQ * H * R * 2
    # QK^T + PV over every (query, visible token) pair; new token i of a
    # sequence sees S - q_len + 1 + i tokens
    attended = int(np.sum(np.maximum(0, inp.seq_lens[:, None].astype(np.int64) - ql + 1
                                     + np.arange(ql)[None, :])))
    flops = 2.0 * attended * H * (R + wl.d_c)
    achieved_gbs = split_bytes / (split_ms * 1e-3) / 1e9
    tflops = flops / (split_ms * 1e-3) / 1e12
    # the binding roof: HBM time of the bytes vs bf16 MFMA time of the flops
    bound = "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > split_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.workload)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.workload)}
    roof.update({"kernel": "k_split (split-KV attention)", "mean_launch_ms": round(split_ms, 5),
                 "launches": n_rec, "algorithmic_bytes_per_launch": split_bytes,
                 "flops_per_launch": flops, "achieved_tflops": round(tflops, 1)})

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.description, "batch": B, "heads": H, "d_c": wl.d_c,
                   "d_rope": wl.d_rope, "seq_len": wl.max_seq_len, "q_len": ql,
                   "total_tokens": total_tokens,
                   "page_size": wl.page_size, "cache": "fp8_e4m3" if wl.fp8 else "bf16",
                   "num_splits": args.num_splits or "auto",
                   "step": ("append_absorb+decode_out(plan,split,merge+W_UV projection)" if ql == 1 else
                            f"append_absorb({ql} new tokens per sequence)+decode_out(plan,split,"
                            f"merge+W_UV projection); value counts the B*q_len new tokens scored")},
        "decode_kernel_tokens_per_s": round(BQ / (split_ms * 1e-3), 1),
        "launch": "hip graph replay of the captured step" if args.graph else "eager calls",
        "settle": settled,
        "roofline": roof,
    }
    if args.graph:
        rec["eager_ms_per_step"] = round(1e3 * eager_elapsed / args.steps, 5)
    if flushed is not None:
        # the whole mla_decode_paged call against the path's algorithmic bytes:
        # cache + q in + o_lat out
        t_med = flushed["median_ms"] * 1e-3
        path_bytes = split_bytes + BQ * H * wl.d_c * 2
        flushed.update({"tokens_per_s": round(BQ / t_med, 1),
                        "achieved_GBs": round(path_bytes / t_med / 1e9, 1),
                        "achieved_tflops": round(flops / t_med / 1e12, 1),
                        "algorithmic_bytes": path_bytes})
        rec["decode_paged_flushed"] = flushed
    if args.cpu_sample > 0:
        rec["cpu_baseline"] = cpu_baseline(inp, min(max(1, args.cpu_sample // ql), B))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
