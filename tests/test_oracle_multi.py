"""Pins of the multi-token-query oracle (`reference_decode_multi`): q_len new
tokens per sequence scored in one pass, each attending causally.

What pins it, other than itself:
* a library routine: torch's scaled_dot_product_attention in fp64 with an
  explicit boolean causal mask over the explicitly materialised per-head K and
  V (query i of q_len sees tokens t <= S - q_len + i; its RoPE position is
  S - q_len + i);
* causality as a property: changing the cached rows after new token i's
  position leaves query i's result unchanged and changes query i + 1's;
* q_len = 1 is single-token decode.
"""
import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, reference_decode, reference_decode_multi, rope,
                    sequence_rows)
from workload import configs, make_inputs

TINY_MTP = configs.TINY.with_(name="tiny_q3", q_len=3)
V2_MTP = configs.V2LITE.with_(name="v2_q4", batch=2, n_heads=4, seq_len=None, seq_lens=(4, 70),
                              q_len=4)


@pytest.mark.parametrize("wl", [TINY_MTP, V2_MTP], ids=lambda w: w.name)
def test_against_torch_sdpa_with_causal_mask(wl):
    inp = make_inputs(wl)
    ref = reference_decode_multi(inp)
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    ql, H = wl.q_len, wl.n_heads
    for b in range(wl.batch):
        C, Kr = sequence_rows(inp, b)
        S = C.shape[0]
        qn = bf16_bits_to_f64(inp.q_nope[b])                  # [ql][H][d_nope]
        qp = bf16_bits_to_f64(inp.q_pe[b])                    # [ql][H][d_rope]
        pos = S - ql + np.arange(ql)
        qr = rope(qp, pos[:, None], wl.rope_base)             # each draft at its own position
        K = np.einsum("sc,hcn->hsn", C, w_uk)                 # [H][S][d_nope]
        V = np.einsum("sc,hcv->hsv", C, w_uv)                 # [H][S][d_v]
        Kf = np.concatenate([K, np.broadcast_to(Kr, (H,) + Kr.shape)], axis=-1)
        Qf = np.concatenate([qn, qr], axis=-1).transpose(1, 0, 2)   # [H][ql][E]
        mask = np.arange(S)[None, :] <= pos[:, None]          # [ql][S]
        got = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(Qf)), torch.from_numpy(np.ascontiguousarray(Kf)),
            torch.from_numpy(np.ascontiguousarray(V)), attn_mask=torch.from_numpy(mask)).numpy()
        exp = ref["out"][b].transpose(1, 0, 2)                # [H][ql][d_v]
        assert np.abs(got - exp).max() <= 1e-12 * max(1.0, np.abs(exp).max())


def test_later_tokens_do_not_reach_earlier_queries():
    wl = TINY_MTP
    inp = make_inputs(wl)
    base = reference_decode_multi(inp, batches=[1])
    b, ql = 1, wl.q_len
    S = int(inp.seq_lens[b])
    s0 = int(inp.cu_seqlens[b])
    for i in range(ql - 1):
        inp2 = make_inputs(wl)
        first_hidden = S - ql + 1 + i                         # first token query i must not see
        inp2.c_kv[s0 + first_hidden:s0 + S] ^= np.uint16(0x4000)   # flip an exponent bit
        got = reference_decode_multi(inp2, batches=[1])
        assert np.array_equal(got["out"][0, i], base["out"][0, i])
        assert not np.allclose(got["out"][0, i + 1], base["out"][0, i + 1])


def test_q_len_one_is_single_token_decode():
    wl = configs.TINY.with_(q_len=1)
    inp = make_inputs(wl)
    single = reference_decode(inp)
    # the same draws viewed with a q_len axis of one
    inp.wl = wl.with_(q_len=1)
    multi = reference_decode_multi(inp)
    assert np.array_equal(multi["out"][:, 0], single["out"])
    assert np.array_equal(multi["lse"][:, 0], single["lse"])
