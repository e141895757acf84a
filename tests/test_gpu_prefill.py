"""mla_prefill_paged on the GPU against the fp64 oracle (`reference_prefill`):
a chunk of new tokens per sequence (the last n_b cached tokens), each
attending causally from its own position, in the explicit form (K and V
up-projected from the latent cache, then dense attention).

Path: append every token -> mla_prefill_paged.  Bar (bf16 inputs, K, V and
P rounded to bf16, fp32 accumulation), over each compared tensor:
max |gpu - oracle| <= 2e-2 and ||gpu - oracle|| / ||oracle|| <= 5e-3; lse
within 1e-2 where finite, -inf exactly where the oracle's is.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_nope_amd as mla
from oracle import reference_prefill
from workload import configs, make_inputs

from gpu_util import assert_close, build_cache, dims_for

pytestmark = pytest.mark.gpu

V3D = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def _wl(name, heads, seq_lens, chunk, page_size=64, fp8=False):
    return configs.V3.with_(name=name, batch=len(seq_lens), n_heads=heads, seq_len=None,
                            seq_lens=tuple(seq_lens), q_len=chunk, page_size=page_size, fp8=fp8)


CASES = [
    # one sequence shorter than the chunk: its first new tokens see nothing
    _wl("v3_h4_c48", 4, (130, 40, 700), 48),
    # several query tiles and ragged key tails, 16-token pages
    _wl("v3_h8_c300_p16", 8, (300, 1000, 257), 300, page_size=16),
    # whole-prompt prefill (the chunk is the whole sequence), 256-token pages
    _wl("v3_h3_prompt_p256", 3, (515,), 515, page_size=256),
    # V2-Lite head count
    configs.V2LITE.with_(name="v2lite_c200", batch=2, seq_len=None, seq_lens=(200, 1100), q_len=200),
    # fp8 E4M3 cache with per-token scales (dequantised as in decode)
    _wl("v3_fp8_h4_c150", 4, (150, 90, 1300), 150, fp8=True),
    _wl("v3_fp8_h2_c64_p16", 2, (64, 33), 64, page_size=16, fp8=True),
]


def run_prefill(inp, d, n_new=None, cache=None, events=None):
    """Packs the last n_new[b] of each sequence's q_len new tokens and runs the
    call; returns host out [T][H][d_v], lse [T][H] and the row offsets."""
    wl = inp.wl
    B, ql, H = wl.batch, wl.q_len, wl.n_heads
    pool, scales, t = cache or build_cache(inp, d)
    n_new = [ql] * B if n_new is None else list(n_new)
    qn = t["q_nope"].reshape(B, ql, H, wl.d_nope)
    qp = t["q_pe"].reshape(B, ql, H, wl.d_rope)
    qn_p = torch.cat([qn[b, ql - n_new[b]:] for b in range(B)]).contiguous()
    qp_p = torch.cat([qp[b, ql - n_new[b]:] for b in range(B)]).contiguous()
    starts = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    q_start = torch.from_numpy(starts).to("cuda")
    out, lse = mla.prefill_paged(d, qn_p, qp_p, q_start, max(n_new), pool, scales,
                                 t["block_table"], t["seq_lens"], t["w_uk"], t["w_uv"], events=events)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    return f(out), f(lse), starts, (pool, scales, t)


def compare(inp, out, lse, starts, n_new=None, heads=None, rows=None):
    wl = inp.wl
    ql = wl.q_len
    n_new = [ql] * wl.batch if n_new is None else list(n_new)
    for b in range(wl.batch):
        if n_new[b] == 0:
            continue
        want = list(range(ql - n_new[b], ql)) if rows is None else [r for r in rows
                                                                    if r >= ql - n_new[b]]
        ref = reference_prefill(inp, batches=[b], heads=heads, rows=want)
        idx = [starts[b] + r - (ql - n_new[b]) for r in want]
        hs = slice(None) if heads is None else list(heads)
        got_o = out[idx][:, hs]
        got_l = lse[idx][:, hs]
        assert_close(got_o, ref["out"][0], f"out[seq {b}]")
        fin = np.isfinite(ref["lse"][0])
        assert np.array_equal(np.isfinite(got_l), fin), f"lse finiteness, seq {b}"
        assert np.all(np.isneginf(got_l[~fin]))
        assert np.max(np.abs(got_l[fin] - ref["lse"][0][fin]), initial=0.0) <= 1e-2


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_prefill_matches_oracle(wl):
    inp = make_inputs(wl)
    print(f"[prefill] {wl.name} H={wl.n_heads} chunk={wl.q_len} seq_lens={list(inp.seq_lens)}",
          flush=True)
    d = dims_for(wl)
    out, lse, starts, _ = run_prefill(inp, d)
    compare(inp, out, lse, starts)
    # new tokens at negative positions: zeros and -inf
    for b in range(wl.batch):
        dead = wl.q_len - int(inp.seq_lens[b])
        if dead > 0:
            rows = slice(starts[b], starts[b] + dead)
            assert np.all(out[rows] == 0) and np.all(np.isneginf(lse[rows]))


def test_ragged_chunks_and_an_empty_one():
    wl = CASES[1]
    inp = make_inputs(wl)
    d = dims_for(wl)
    n_new = [300, 129, 0]
    print(f"[prefill] ragged n_new={n_new}", flush=True)
    out, lse, starts, _ = run_prefill(inp, d, n_new)
    assert out.shape[0] == sum(n_new)
    compare(inp, out, lse, starts, n_new)


def test_rows_outside_the_chunk_are_untouched():
    # rows past max_q_len of a longer chunk are not computed; the output
    # buffer keeps what it held there
    wl = _wl("v3_h2_c40", 2, (90,), 40)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    qn = t["q_nope"].reshape(40, 2, 128).contiguous()
    qp = t["q_pe"].reshape(40, 2, 64).contiguous()
    q_start = torch.tensor([0, 40], dtype=torch.int32, device="cuda")
    out = torch.full((40, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    mla.prefill_paged(d, qn, qp, q_start, 32, pool, scales, t["block_table"], t["seq_lens"],
                      t["w_uk"], t["w_uv"], out=out, want_lse=False)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    assert np.all(o[32:] == 7.0)
    ref = reference_prefill(inp, rows=list(range(32)))
    assert_close(o[:32], ref["out"][0], "out")


def test_full_size_sampled():
    """The benchmarked chunk: DeepSeek-V3 shape, 2 sequences of 8192 tokens,
    the second 4096-token chunk of each (H = 128, page 64); sampled rows and
    heads against the oracle."""
    wl = configs.V3.with_(name="v3prefill", batch=2, seq_len=8192, q_len=4096)
    inp = make_inputs(wl)
    d = dims_for(wl)
    print("[prefill] full size B=2 S=8192 chunk=4096 H=128", flush=True)
    out, lse, starts, _ = run_prefill(inp, d)
    compare(inp, out, lse, starts, heads=[0, 77, 127], rows=[0, 1, 127, 128, 2047, 4095])


def test_rows_before_the_buffer_are_skipped():
    # q_start[0] = -5: the chunk's first five rows lie outside [0, T) and are
    # neither read nor written; the other rows keep their positions
    wl = _wl("v3_h2_c25", 2, (70,), 25)
    inp = make_inputs(wl)
    d = dims_for(wl)
    pool, scales, t = build_cache(inp, d)
    qn = t["q_nope"].reshape(25, 2, 128)[5:].contiguous()
    qp = t["q_pe"].reshape(25, 2, 64)[5:].contiguous()
    q_start = torch.tensor([-5, 20], dtype=torch.int32, device="cuda")
    out = torch.full((20, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((20, 2), 3.0, dtype=torch.float32, device="cuda")
    mla.prefill_paged(d, qn, qp, q_start, 25, pool, scales, t["block_table"], t["seq_lens"],
                      t["w_uk"], t["w_uv"], out=out, lse=lse)
    torch.cuda.synchronize()
    ref = reference_prefill(inp, rows=list(range(5, 25)))
    assert_close(out.float().cpu().numpy().astype(np.float64), ref["out"][0], "out")
    assert np.max(np.abs(lse.cpu().numpy() - ref["lse"][0])) <= 1e-2


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("amp", [192.0, 1664.0], ids=["jump20", "jump173"])
def test_late_key_raises_the_offset(amp, fp8):
    # One key (t* = 150, key tile 4) scores softmax_scale * amp: W_UK[h] maps
    # q_nope = amp e_0 onto latent column 0 (column 0 of W_UK[h] is e_0), and
    # c_kv column 0 is 0 except 1 at t*.  For a query that sees t*, that tile's
    # maximum exceeds the offset set by the earlier key tiles (all scores 0) by
    # amp * softmax_scale * log2(e) = 20 or 173 (base 2): the running offset
    # moves and the earlier O and denominator are rescaled (by 2^-20, or to 0).
    # Queries before t* see only zero scores.
    wl = _wl("v3_h4_c120_star", 4, (300,), 120, fp8=fp8)
    inp = make_inputs(wl)
    from workload import f32_to_bf16_bits
    from oracle import bf16_bits_to_f64
    c = inp.c_kv.copy()
    if fp8:
        # every row's largest magnitude is exactly 7 (column 1), so each scale
        # is 2^-6 and the dequantised rows are exact in bf16: the huge score
        # carries no rounding of its key
        c = f32_to_bf16_bits(np.clip(bf16_bits_to_f64(c), -6.5, 6.5).astype(np.float32))
        c[:, 1] = 0x40E0                                   # 7.0
        inp.k_pe = f32_to_bf16_bits(np.clip(bf16_bits_to_f64(inp.k_pe), -4.5, 4.5).astype(np.float32))
    c[:, 0] = 0
    c[150, 0] = 0x3F80                                     # 1.0
    inp.c_kv = c
    w = inp.w_uk.copy()
    w[:, :, 0] = 0
    w[:, 0, 0] = 0x3F80                                    # column 0 of W_UK[h] = e_0
    inp.w_uk = w
    qn = np.zeros_like(inp.q_nope)
    qn[..., 0] = f32_to_bf16_bits(np.array([amp], np.float32))[0]
    inp.q_nope = qn
    inp.q_pe = np.zeros_like(inp.q_pe)
    d = dims_for(wl)
    print(f"[prefill star] amp={amp} fp8={fp8}", flush=True)
    out, lse, starts, _ = run_prefill(inp, d)
    compare(inp, out, lse, starts)
