"""Pins for the oracle's attention (CPU only).

* explicit (un-absorbed) form == absorbed form, by associativity of matrix
  products ("DeepSeek-V2拆解" (sheratonhq.com) §2.1; zskr.cn §2.2);
* softmax rows sum to 1;
* a library routine: torch's scaled_dot_product_attention in fp64 over the
  explicitly materialised per-head K and V (its default scale is
  1/sqrt(query width) = 1/sqrt(d_nope + d_rope));
* special cases with closed forms: S = 1 (a GEMV), q = 0 (the mean), q_pe = 0
  (k_pe drops out), a delta query (one token picked), S = 0.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import (absorb_query, bf16_bits_to_f64, cache_rows, decode_absorbed,
                    decode_explicit, latent_attention, rope, softmax_with_lse)
from workload import configs, make_inputs


def _seq(inp, b):
    return oracle.sequence_rows(inp, b)


def _weights(inp):
    return bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)


SMALL_V2 = configs.V2LITE.with_(name="v2small", batch=2, n_heads=4, seq_len=None,
                                seq_lens=(1, 77), page_size=64)


@pytest.mark.parametrize("wl", [configs.TINY, SMALL_V2], ids=lambda w: w.name)
def test_explicit_equals_absorbed(wl):
    inp = make_inputs(wl)
    w_uk, w_uv = _weights(inp)
    for b in range(wl.batch):
        C, Kr = _seq(inp, b)
        qn, qp = bf16_bits_to_f64(inp.q_nope[b]), bf16_bits_to_f64(inp.q_pe[b])
        S = int(inp.seq_lens[b])
        e = decode_explicit(qn, qp, C, Kr, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
        a = decode_absorbed(qn, qp, C, Kr, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
        for x, y in zip(e, a):
            assert np.linalg.norm(x - y) <= 1e-12 * np.linalg.norm(y)


def test_softmax_rows_sum_to_one():
    s = np.random.default_rng(0).standard_normal((7, 1000)) * 30
    p, lse = softmax_with_lse(s)
    assert np.all(np.abs(p.sum(-1) - 1) <= 1e-12)
    assert np.allclose(lse, np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1))


@pytest.mark.parametrize("wl", [configs.TINY, SMALL_V2], ids=lambda w: w.name)
def test_against_torch_sdpa(wl):
    inp = make_inputs(wl)
    w_uk, w_uv = _weights(inp)
    for b in range(wl.batch):
        C, Kr = _seq(inp, b)
        S = int(inp.seq_lens[b])
        qn, qp = bf16_bits_to_f64(inp.q_nope[b]), bf16_bits_to_f64(inp.q_pe[b])
        out, lse, o_lat = decode_explicit(qn, qp, C, Kr, w_uk, w_uv, S - 1,
                                          wl.softmax_scale, wl.rope_base)
        H = wl.n_heads
        Q = np.concatenate([qn, rope(qp, S - 1, wl.rope_base)], -1)[:, None, :]   # [H][1][E]
        K = np.concatenate([np.matmul(C[None], w_uk), np.broadcast_to(Kr, (H,) + Kr.shape)], -1)
        V = np.matmul(C[None], w_uv)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(np.ascontiguousarray(K)),
            torch.from_numpy(np.ascontiguousarray(V))).numpy()[:, 0, :]
        assert np.abs(out - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_single_token_is_gemv():
    inp = make_inputs(SMALL_V2)
    w_uk, w_uv = _weights(inp)
    C, Kr = _seq(inp, 0)
    assert C.shape[0] == 1
    qn, qp = bf16_bits_to_f64(inp.q_nope[0]), bf16_bits_to_f64(inp.q_pe[0])
    out, lse, o_lat = decode_explicit(qn, qp, C, Kr, w_uk, w_uv, 0, 0.1, 1e4)
    for h in range(SMALL_V2.n_heads):
        assert np.allclose(out[h], w_uv[h].T @ C[0], rtol=1e-13, atol=1e-15)
    assert np.array_equal(o_lat, np.broadcast_to(C[0], o_lat.shape))


def test_zero_query_gives_mean_and_log_s():
    inp = make_inputs(configs.TINY)
    w_uk, w_uv = _weights(inp)
    C, Kr = _seq(inp, 1)
    H = configs.TINY.n_heads
    z = np.zeros((H, configs.TINY.d_nope)), np.zeros((H, configs.TINY.d_rope))
    out, lse, o_lat = decode_explicit(z[0], z[1], C, Kr, w_uk, w_uv, 63, 0.3, 1e4)
    for h in range(H):
        assert np.allclose(out[h], w_uv[h].T @ C.mean(0), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, np.log(C.shape[0]), rtol=1e-14)


def test_zero_qpe_makes_kpe_irrelevant():
    wl = configs.TINY
    inp = make_inputs(wl)
    w_uk, w_uv = _weights(inp)
    qn = bf16_bits_to_f64(inp.q_nope[1])
    qp = np.zeros((wl.n_heads, wl.d_rope))
    S = int(inp.seq_lens[1])
    s0, s1 = int(inp.cu_seqlens[1]), int(inp.cu_seqlens[2])
    C, Kr = cache_rows(inp.c_kv[s0:s1], inp.k_pe[s0:s1], np.arange(S), wl.rope_base, False)
    C2, Kr2 = cache_rows(inp.c_kv[s0:s1], inp.k_pe[s0:s1] ^ np.uint16(0x1234), np.arange(S),
                         wl.rope_base, False)
    a = decode_explicit(qn, qp, C, Kr, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
    b = decode_explicit(qn, qp, C2, Kr2, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
    assert not np.allclose(Kr, Kr2)
    assert np.array_equal(a[0], b[0])
    # while a nonzero q_pe does see k_pe
    qp1 = bf16_bits_to_f64(inp.q_pe[1])
    c = decode_explicit(qn, qp1, C, Kr, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
    d = decode_explicit(qn, qp1, C2, Kr2, w_uk, w_uv, S - 1, wl.softmax_scale, wl.rope_base)
    assert not np.allclose(c[0], d[0])


def test_delta_query_picks_one_token():
    rng = np.random.default_rng(4)
    S, d_c, d_r, H = 50, 32, 16, 3
    C = rng.standard_normal((S, d_c))
    Kr = rng.standard_normal((S, d_r))
    C[:, 0] = 0.0
    t_star = 17
    C[t_star, 0] = 1.0
    q = np.zeros((H, d_c + d_r))
    q[:, 0] = 500.0
    o_lat, lse = latent_attention(q, C, Kr, scale=1.0)
    assert np.array_equal(o_lat, np.broadcast_to(C[t_star], o_lat.shape))
    assert np.allclose(lse, 500.0)


def test_empty_sequence():
    H, d = 2, 8
    out, lse, o_lat = decode_explicit(np.ones((H, 4)), np.ones((H, 4)), np.zeros((0, d)),
                                      np.zeros((0, 4)), np.ones((H, d, 4)), np.ones((H, d, 4)),
                                      -1, 0.5, 1e4)
    assert np.all(out == 0) and np.all(o_lat == 0) and np.all(np.isneginf(lse))


def test_absorb_query_shapes_and_rope_position():
    wl = configs.TINY
    inp = make_inputs(wl)
    w_uk, _ = _weights(inp)
    qn, qp = bf16_bits_to_f64(inp.q_nope), bf16_bits_to_f64(inp.q_pe)
    q = absorb_query(qn, qp, w_uk, inp.q_pos(), wl.rope_base)
    assert q.shape == (wl.batch, wl.n_heads, wl.d_c + wl.d_rope)
    for b in range(wl.batch):
        for h in range(wl.n_heads):
            assert np.allclose(q[b, h, :wl.d_c], w_uk[h] @ qn[b, h], rtol=1e-14, atol=1e-15)
            assert np.allclose(q[b, h, wl.d_c:], rope(qp[b, h], inp.seq_lens[b] - 1, wl.rope_base))
