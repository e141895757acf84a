"""Pins of the explicit-form prefill oracle (`prefill_explicit`,
`reference_prefill`): a chunk of new tokens per sequence, the last q_len
cached ones, each attending causally from its own position.

What pins it, other than itself:
* a library routine: torch's scaled_dot_product_attention in fp64 with an
  explicit boolean mask over independently materialised per-head K and V;
* single-query decode: every row equals `decode_explicit` over the row's
  visible prefix (pinned on its own by the associativity and SDPA checks);
* a closed form: in a whole-prompt chunk the first token sees only token 0,
  so its output is V_h[0] = C[0] @ W_UV[h] and its lse is its one score;
* causality as a property: rows after a query's position never reach it;
* a chunk of at most 16 tokens is the multi-token-query oracle.
"""
import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, decode_explicit, prefill_explicit, reference_decode_multi,
                    reference_prefill, rope, sequence_rows)
from workload import configs, make_inputs

# second sequence shorter than the chunk: its first 8 new tokens see nothing
V3_SMALL = configs.V3.with_(name="v3_pf", batch=2, n_heads=3, seq_len=None, seq_lens=(130, 40),
                            q_len=48)
TINY_PF = configs.TINY.with_(name="tiny_pf", q_len=12)


@pytest.mark.parametrize("wl", [V3_SMALL, TINY_PF], ids=lambda w: w.name)
def test_against_torch_sdpa_with_explicit_mask(wl):
    inp = make_inputs(wl)
    ref = reference_prefill(inp)
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    ql, H = wl.q_len, wl.n_heads
    for b in range(wl.batch):
        C, Kr = sequence_rows(inp, b)
        S = C.shape[0]
        pos = S - ql + np.arange(ql)
        live = pos >= 0
        qn = bf16_bits_to_f64(inp.q_nope[b])[live]              # [n][H][d_nope]
        qr = rope(bf16_bits_to_f64(inp.q_pe[b])[live], pos[live][:, None], wl.rope_base)
        K = np.stack([C @ w_uk[h] for h in range(H)])            # [H][S][d_nope]
        V = np.stack([C @ w_uv[h] for h in range(H)])            # [H][S][d_v]
        Kf = np.concatenate([K, np.broadcast_to(Kr, (H,) + Kr.shape)], axis=-1)
        Qf = np.concatenate([qn, qr], axis=-1).transpose(1, 0, 2)
        mask = np.arange(S)[None, :] <= pos[live][:, None]
        got = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(Qf)), torch.from_numpy(np.ascontiguousarray(Kf)),
            torch.from_numpy(np.ascontiguousarray(V)), attn_mask=torch.from_numpy(mask),
            scale=wl.softmax_scale).numpy()
        exp = ref["out"][b][live].transpose(1, 0, 2)
        assert np.abs(got - exp).max() <= 1e-12 * max(1.0, np.abs(exp).max())
        # tokens with no visible row: zeros and -inf
        assert np.all(ref["out"][b][~live] == 0) and np.all(np.isneginf(ref["lse"][b][~live]))


def test_rows_are_single_query_decode_over_their_prefix():
    wl = V3_SMALL
    inp = make_inputs(wl)
    rows = [8, 9, 30, 47]
    ref = reference_prefill(inp, rows=rows)
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    for n, b in enumerate(range(wl.batch)):
        C, Kr = sequence_rows(inp, b)
        S = C.shape[0]
        for k, i in enumerate(rows):
            L = S - wl.q_len + 1 + i
            qn = bf16_bits_to_f64(inp.q_nope[b][i])
            qp = bf16_bits_to_f64(inp.q_pe[b][i])
            o, l, _ = decode_explicit(qn, qp, C[:L], Kr[:L], w_uk, w_uv, L - 1, wl.softmax_scale,
                                      wl.rope_base)
            assert np.abs(ref["out"][n, k] - o).max() <= 1e-12
            assert np.abs(ref["lse"][n, k] - l).max() <= 1e-12


def test_whole_prompt_first_token_is_its_value_row():
    wl = configs.V3.with_(name="v3_prompt", batch=1, n_heads=2, seq_len=None, seq_lens=(20,),
                          q_len=20)
    inp = make_inputs(wl)
    ref = reference_prefill(inp, rows=[0])
    C, Kr = sequence_rows(inp, 0)
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    qn = bf16_bits_to_f64(inp.q_nope[0][0])
    qp = bf16_bits_to_f64(inp.q_pe[0][0])
    for h in range(wl.n_heads):
        assert np.abs(ref["out"][0, 0, h] - C[0] @ w_uv[h]).max() <= 1e-12
        # position 0: RoPE is the identity there
        s = wl.softmax_scale * (qn[h] @ (C[0] @ w_uk[h]) + qp[h] @ Kr[0])
        assert abs(ref["lse"][0, 0, h] - s) <= 1e-12


def test_later_rows_do_not_reach_earlier_queries():
    wl = V3_SMALL.with_(n_heads=2)
    inp = make_inputs(wl)
    b, i = 0, 20
    S = int(inp.seq_lens[b])
    p = S - wl.q_len + i
    w_uk, w_uv = bf16_bits_to_f64(inp.w_uk), bf16_bits_to_f64(inp.w_uv)
    C, Kr = sequence_rows(inp, b)
    qn = bf16_bits_to_f64(inp.q_nope[b])
    qp = bf16_bits_to_f64(inp.q_pe[b])
    pos = S - wl.q_len + np.arange(wl.q_len)
    o1, _ = prefill_explicit(qn, qp, C, Kr, w_uk, w_uv, pos, wl.softmax_scale, wl.rope_base)
    C2, Kr2 = C.copy(), Kr.copy()
    C2[p + 1:] = -C2[p + 1:] * 3.0
    Kr2[p + 1:] = 7.0
    o2, _ = prefill_explicit(qn, qp, C2, Kr2, w_uk, w_uv, pos, wl.softmax_scale, wl.rope_base)
    assert np.array_equal(o1[: i + 1], o2[: i + 1])
    assert np.abs(o1[i + 1] - o2[i + 1]).max() > 1e-3


def test_short_chunk_is_the_multi_token_query():
    wl = TINY_PF
    inp = make_inputs(wl)
    a = reference_prefill(inp)
    m = reference_decode_multi(inp)
    assert np.abs(a["out"] - m["out"]).max() <= 1e-12
    fin = np.isfinite(m["lse"])
    assert np.array_equal(np.isfinite(a["lse"]), fin)
    assert np.abs(a["lse"][fin] - m["lse"][fin]).max() <= 1e-12
