"""Plain, slow fp64 CPU oracle for Multi-head Latent Attention (MLA) decode
(single and multi-token queries), the down-projection into the latent, and
prefill in the explicit form.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import, call or execute anything under oracle/.  It shares no
code with the HIP path and never imports it; it takes plain numpy arrays
(bf16 inputs as uint16 bit patterns) and returns float64 arrays.

What MLA decode computes, and where the pages state it
-------------------------------------------------------
* Only a low-rank joint latent c_t (width d_c) is cached per token; K and V
  are recovered from it by per-head up-projections W_UK and W_UV.
  ("DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%" (sheratonhq.com) §2.1;
  "当MoE遇见MLA，推理效率的'黄金搭档'" (agent.csdn.net) §2.1.)
* Position information rides in a separate decoupled-RoPE branch, because RoPE
  does not commute with the low-rank up-projection (sheratonhq.com §2.1;
  zskr.cn "LLM推理优化的新范式：从内存墙到计算墙的跨越" §2.1).  The rotated
  key part k_pe is shared by all heads; each head has its own q_pe.
* The latent of the current token is appended to the cache before it is used
  (the cat-then-return in sheratonhq.com §2.1's compression sketch), so the
  query of sequence b sits at position S_b - 1 and sees all S_b cached tokens.
* W_UK can be folded into the query side and W_UV into the output side
  (sheratonhq.com §2.1; zskr.cn §2.2, reordering by associativity of matrix
  products).  `decode_explicit` below is the un-absorbed form the pages start
  from; `decode_absorbed` is the reordered form, kept here only so a test can
  check that the two agree.

Readings where the pages are silent (each listed in the design notes):
  RoPE = RoFormer's rotation of consecutive pairs (2i, 2i+1) by angle
  pos * base^(-2i/d_rope); K_h = C @ W_UK[h] with W_UK[h] of shape (d_c, d_nope);
  V_h = C @ W_UV[h] with W_UV[h] of shape (d_c, d_v); the softmax scale
  multiplies the whole score (nope and rope parts); V uses only the c_kv part
  of the cached row; fp8 caches keep one fp32 scale per token = absmax / 448
  over the whole (c_kv || rotated k_pe) row.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode_satfinite, f64_to_bf16_bits, E4M3_MAX


# ----------------------------------------------------------------------------
# Cache size (sheratonhq.com §2.1 and §4.2: MHA caches 2*n_h*d_h*l elements,
# MLA caches d_c*l; here the MLA row also holds the d_rope-wide rotated key).
# ----------------------------------------------------------------------------
def mha_cache_elements_per_token(layers: int, n_heads: int, head_dim: int) -> int:
    return layers * 2 * n_heads * head_dim


def mla_cache_elements_per_token(layers: int, d_c: int, d_rope: int) -> int:
    return layers * (d_c + d_rope)


def mla_cache_bytes_per_token(d_c: int, d_rope: int, fp8: bool) -> int:
    """One layer: bf16 rows are 2 bytes per element; fp8 rows are 1 byte per
    element plus one fp32 scale."""
    return (d_c + d_rope) + 4 if fp8 else 2 * (d_c + d_rope)


# ----------------------------------------------------------------------------
# Down-projection of the hidden state into the cached latent
# ----------------------------------------------------------------------------
def project_latent(h_bits: np.ndarray, w_down_bits: np.ndarray, d_c: int):
    """c_kv and the un-rotated key RoPE part of new tokens from their hidden
    states: the latent is the down-projection of h ("DeepSeek-V2拆解" §2.1:
    `down_proj = nn.Linear(d_model, kv_rank)`, c_kv = down_proj(h), then
    appended to the cache); the RoPE key comes from h through its own
    projection in the decoupled branch (same section).  Reading: one weight
    w_down [d_c + d_rope][d_model] in nn.Linear layout (output rows), W_DKV in
    rows [0, d_c) and W_KR in rows [d_c, d_c + d_rope); y = h . w_down^T
    exactly, rounded once to bf16.  Returns (c_kv bits [T][d_c], k_pe bits
    [T][d_rope]) as uint16, ready for `cache_rows`."""
    h = bf16_bits_to_f64(h_bits)
    w = bf16_bits_to_f64(w_down_bits)
    y = h @ w.T
    bits = f64_to_bf16_bits(y)
    return bits[:, :d_c], bits[:, d_c:]


# ----------------------------------------------------------------------------
# RoPE (reading: RoFormer, consecutive pairs)
# ----------------------------------------------------------------------------
def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of x (even width d) by position `pos`.

    Pair i = (x[2i], x[2i+1]) turns by angle pos * base**(-2i/d):
        y[2i]   = x[2i] cos - x[2i+1] sin
        y[2i+1] = x[2i] sin + x[2i+1] cos
    `pos` broadcasts against x's leading axes.  All in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# ----------------------------------------------------------------------------
# What the cache holds for each token
# ----------------------------------------------------------------------------
def fp8_quantize_rows(rows_f32: np.ndarray):
    """Per-token fp8 encoding of float32 rows (reading: one scale per row).

    scale = fp32(absmax / 448) with an IEEE fp32 division; code = E4M3FN of the
    fp32 quotient row/scale, rounded to nearest even and clamped to +-448.  A
    row of zeros gets scale 0 and all-zero codes.  Returns (codes uint8, scale f32).
    """
    r = np.asarray(rows_f32, dtype=np.float32)
    absmax = np.max(np.abs(r), axis=-1)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (r / safe[..., None]).astype(np.float32)
    codes = e4m3fn_encode_satfinite(q)
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def fp8_cache_codes(c_kv_bits: np.ndarray, k_pe_bits: np.ndarray, positions: np.ndarray,
                    base: float):
    """The fp8 cache content of a run of tokens: the row (c_kv || RoPE(k_pe))
    rounded to fp32, then `fp8_quantize_rows`.  Returns (codes [T][R], scale [T])."""
    C = bf16_bits_to_f64(c_kv_bits)
    Kr = rope(bf16_bits_to_f64(k_pe_bits), positions, base)
    row = np.concatenate([C, Kr], axis=-1).astype(np.float32)
    return fp8_quantize_rows(row)


def cache_rows(c_kv_bits: np.ndarray, k_pe_bits: np.ndarray, positions: np.ndarray,
               base: float, fp8: bool):
    """Mathematical content of the cached rows for a run of tokens.

    c_kv_bits [T][d_c] and k_pe_bits [T][d_rope] are bf16 inputs; positions [T].
    Returns (C [T][d_c], Kr [T][d_rope]) in float64: C is the latent, Kr the key
    RoPE part rotated at its own position.  For an fp8 cache the row (C || Kr)
    is first rounded to fp32, encoded as above and decoded back (code * scale).
    """
    if fp8:
        codes, scale = fp8_cache_codes(c_kv_bits, k_pe_bits, positions, base)
        deq = e4m3fn_decode(codes) * scale.astype(np.float64)[..., None]
        d_c = c_kv_bits.shape[-1]
        return deq[..., :d_c], deq[..., d_c:]
    C = bf16_bits_to_f64(c_kv_bits)
    Kr = rope(bf16_bits_to_f64(k_pe_bits), positions, base)
    return C, Kr


# ----------------------------------------------------------------------------
# Softmax attention of one query row per head over the cached sequence
# ----------------------------------------------------------------------------
def softmax_with_lse(s: np.ndarray):
    """Row softmax over the last axis and its natural-log normaliser."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def decode_explicit(q_nope: np.ndarray, q_pe: np.ndarray, C: np.ndarray, Kr: np.ndarray,
                    w_uk: np.ndarray, w_uv: np.ndarray, q_pos: int, scale: float,
                    base: float, heads=None):
    """Un-absorbed MLA decode for one sequence.

    q_nope [H][d_nope], q_pe [H][d_rope] (float64, un-rotated); C [S][d_c] and
    Kr [S][d_rope] from `cache_rows`; w_uk [H][d_c][d_nope], w_uv [H][d_c][d_v].
    For each head h: K_h = C @ W_UK[h], V_h = C @ W_UV[h] are materialised,
    s_t = scale * (q_nope[h] . K_h[t] + RoPE(q_pe[h], q_pos) . Kr[t]),
    p = softmax(s), out[h] = p @ V_h.  Also returns lse[h] and the latent output
    o_lat[h] = p @ C (the quantity the absorbed kernel produces before W_UV).
    S = 0 gives out = o_lat = 0 and lse = -inf.
    """
    H = q_nope.shape[0]
    heads = range(H) if heads is None else heads
    heads = list(heads)
    d_c, d_v = C.shape[1], w_uv.shape[2]
    S = C.shape[0]
    out = np.zeros((len(heads), d_v))
    o_lat = np.zeros((len(heads), d_c))
    lse = np.full(len(heads), -np.inf)
    if S == 0:
        return out, lse, o_lat
    qr = rope(q_pe[heads], q_pos, base)                       # [h][d_rope]
    chunk = 8
    for j0 in range(0, len(heads), chunk):
        hs = heads[j0:j0 + chunk]
        K = np.matmul(C[None], w_uk[hs])                       # [hc][S][d_nope]
        V = np.matmul(C[None], w_uv[hs])                       # [hc][S][d_v]
        s = np.einsum("hsd,hd->hs", K, q_nope[hs]) + np.einsum("sd,hd->hs", Kr, qr[j0:j0 + len(hs)])
        p, l = softmax_with_lse(scale * s)
        out[j0:j0 + len(hs)] = np.einsum("hs,hsv->hv", p, V)
        o_lat[j0:j0 + len(hs)] = p @ C
        lse[j0:j0 + len(hs)] = l
    return out, lse, o_lat


# ----------------------------------------------------------------------------
# The absorbed (reordered) form, step by step.  Used as per-step references for
# the three kernels' parity tests and by the associativity check.
# ----------------------------------------------------------------------------
def absorb_query(q_nope: np.ndarray, q_pe: np.ndarray, w_uk: np.ndarray, q_pos, base: float):
    """q[h] = (W_UK[h] @ q_nope[h]) || RoPE(q_pe[h], q_pos): the latent-space
    query (q_nope folded through W_UK) next to the rotated RoPE query.
    Shapes: q_nope [..., H, d_nope], q_pe [..., H, d_rope]; q_pos broadcasts over
    the leading axes.  Returns [..., H, d_c + d_rope]."""
    q_lat = np.einsum("hcn,...hn->...hc", w_uk, q_nope)
    pos = np.asarray(q_pos, dtype=np.float64)[..., None]       # one position per row of heads
    q_rot = rope(q_pe, pos, base)
    return np.concatenate([q_lat, q_rot], axis=-1)


def latent_attention(q: np.ndarray, C: np.ndarray, Kr: np.ndarray, scale: float):
    """Single-query softmax attention in the latent space for one sequence:
    keys are the cached rows (C || Kr), values are C.  q [H][d_c + d_rope].
    Returns (o_lat [H][d_c], lse [H]); S = 0 gives zeros and -inf."""
    H = q.shape[0]
    if C.shape[0] == 0:
        return np.zeros((H, C.shape[1])), np.full(H, -np.inf)
    rows = np.concatenate([C, Kr], axis=-1)                   # [S][d_c + d_rope]
    p, lse = softmax_with_lse(scale * (q @ rows.T))
    return p @ C, lse


def out_projection(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """out[..., h, :] = W_UV[h]^T @ o_lat[..., h, :] (W_UV folded on the output side)."""
    return np.einsum("hcv,...hc->...hv", w_uv, o_lat)


def decode_absorbed(q_nope, q_pe, C, Kr, w_uk, w_uv, q_pos, scale, base):
    q = absorb_query(q_nope, q_pe, w_uk, q_pos, base)
    o_lat, lse = latent_attention(q, C, Kr, scale)
    return out_projection(o_lat, w_uv), lse, o_lat


# ----------------------------------------------------------------------------
# Whole batches from the seeded inputs
# ----------------------------------------------------------------------------
def sequence_rows(inp, b: int):
    """(C, Kr) of sequence b of a generated workload (see workload.generate)."""
    wl = inp.wl
    s0, s1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
    pos = np.arange(s1 - s0)
    return cache_rows(inp.c_kv[s0:s1], inp.k_pe[s0:s1], pos, wl.rope_base, wl.fp8)


def reference_decode(inp, batches=None, heads=None):
    """Explicit-form oracle over (a subset of) a generated batch.

    Returns dict with out [nb][nh][d_v], lse [nb][nh], o_lat [nb][nh][d_c]
    for the requested sequences and heads (default: all)."""
    wl = inp.wl
    B, H = len(inp.seq_lens), wl.n_heads
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    w_uk = bf16_bits_to_f64(inp.w_uk)
    w_uv = bf16_bits_to_f64(inp.w_uv)
    out = np.zeros((len(batches), len(heads), wl.d_v))
    o_lat = np.zeros((len(batches), len(heads), wl.d_c))
    lse = np.zeros((len(batches), len(heads)))
    for i, b in enumerate(batches):
        C, Kr = sequence_rows(inp, b)
        qn = bf16_bits_to_f64(inp.q_nope[b])
        qp = bf16_bits_to_f64(inp.q_pe[b])
        o, l, ol = decode_explicit(qn, qp, C, Kr, w_uk, w_uv, int(inp.seq_lens[b]) - 1,
                                   wl.softmax_scale, wl.rope_base, heads)
        out[i], lse[i], o_lat[i] = o, l, ol
    return {"out": out, "lse": lse, "o_lat": o_lat}


def reference_decode_multi(inp, batches=None, heads=None):
    """Explicit-form oracle for q_len > 1 new tokens per sequence, scored in one
    pass (the verification of multi-token-prediction drafts: "deepseek.csdn.net"
    section 6).  Reading: the q_len new tokens are the last q_len cached tokens
    of each sequence, and new token i (0-based) attends causally, to the first
    L = S_b - q_len + 1 + i tokens, from position L - 1.  Each query is
    `decode_explicit` over that prefix.

    Returns dict with out [nb][q_len][nh][d_v], lse [nb][q_len][nh] and
    o_lat [nb][q_len][nh][d_c]."""
    wl = inp.wl
    ql = wl.q_len
    B, H = len(inp.seq_lens), wl.n_heads
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    w_uk = bf16_bits_to_f64(inp.w_uk)
    w_uv = bf16_bits_to_f64(inp.w_uv)
    out = np.zeros((len(batches), ql, len(heads), wl.d_v))
    o_lat = np.zeros((len(batches), ql, len(heads), wl.d_c))
    lse = np.zeros((len(batches), ql, len(heads)))
    for n, b in enumerate(batches):
        C, Kr = sequence_rows(inp, b)
        S = int(inp.seq_lens[b])
        qn = bf16_bits_to_f64(inp.q_nope[b]).reshape(ql, H, wl.d_nope)
        qp = bf16_bits_to_f64(inp.q_pe[b]).reshape(ql, H, wl.d_rope)
        for i in range(ql):
            L = max(0, S - ql + 1 + i)
            o, l, ol = decode_explicit(qn[i], qp[i], C[:L], Kr[:L], w_uk, w_uv, L - 1,
                                       wl.softmax_scale, wl.rope_base, heads)
            out[n, i], lse[n, i], o_lat[n, i] = o, l, ol
    return {"out": out, "lse": lse, "o_lat": o_lat}


# ----------------------------------------------------------------------------
# Prefill in the explicit form
# ----------------------------------------------------------------------------
def prefill_explicit(q_nope: np.ndarray, q_pe: np.ndarray, C: np.ndarray, Kr: np.ndarray,
                     w_uk: np.ndarray, w_uv: np.ndarray, q_pos: np.ndarray, scale: float,
                     base: float, heads=None):
    """Causal attention of n new tokens of one sequence in the un-absorbed form.

    Reordering by associativity pays off in decode; in prefill it lowers the
    arithmetic intensity (zskr.cn "LLM推理优化的新范式：从内存墙到计算墙的跨越"
    §2.2, the per-stage table), so prefill keeps the explicit form: K_h = C @
    W_UK[h] and V_h = C @ W_UV[h] are materialised from the cached latent, and
    query i (position q_pos[i]) attends to the tokens t <= q_pos[i] with
    s_t = scale * (q_nope[i][h] . K_h[t] + RoPE(q_pe[i][h], q_pos[i]) . Kr[t]).

    q_nope [n][H][d_nope], q_pe [n][H][d_rope] (float64, un-rotated); C [S][d_c],
    Kr [S][d_rope] from `cache_rows`; q_pos int [n].  Returns out [n][nh][d_v]
    and lse [n][nh]; a query with no visible token (q_pos < 0) gives out = 0 and
    lse = -inf.
    """
    n, H = q_nope.shape[0], q_nope.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    d_v = w_uv.shape[2]
    S = C.shape[0]
    q_pos = np.asarray(q_pos, dtype=np.int64)
    out = np.zeros((n, len(heads), d_v))
    lse = np.full((n, len(heads)), -np.inf)
    if S == 0 or n == 0:
        return out, lse
    visible = np.arange(S)[None, :] <= q_pos[:, None]            # [n][S]
    live = visible.any(axis=1)
    qr = rope(q_pe[:, heads], q_pos[:, None], base)             # [n][nh][d_rope]
    for j, h in enumerate(heads):
        K = C @ w_uk[h]                                           # [S][d_nope]
        V = C @ w_uv[h]                                           # [S][d_v]
        s = scale * (q_nope[:, h] @ K.T + qr[:, j] @ Kr.T)        # [n][S]
        s = np.where(visible, s, -np.inf)
        p, l = softmax_with_lse(s[live])
        out[live, j] = p @ V
        lse[live, j] = l
    return out, lse


def reference_prefill(inp, batches=None, heads=None, rows=None):
    """`prefill_explicit` over (a subset of) a generated batch whose q_len new
    tokens per sequence are the last q_len cached ones: new token i of
    sequence b sits at position S_b - q_len + i (the reading used for the
    multi-token query, extended to a whole chunk).  `rows` picks new tokens
    (default: all).  Returns out [nb][nr][nh][d_v] and lse [nb][nr][nh]."""
    wl = inp.wl
    ql, H = wl.q_len, wl.n_heads
    B = len(inp.seq_lens)
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    rows = list(range(ql)) if rows is None else list(rows)
    w_uk = bf16_bits_to_f64(inp.w_uk)
    w_uv = bf16_bits_to_f64(inp.w_uv)
    out = np.zeros((len(batches), len(rows), len(heads), wl.d_v))
    lse = np.zeros((len(batches), len(rows), len(heads)))
    for n, b in enumerate(batches):
        C, Kr = sequence_rows(inp, b)
        S = int(inp.seq_lens[b])
        qn = bf16_bits_to_f64(inp.q_nope[b]).reshape(ql, H, wl.d_nope)[rows]
        qp = bf16_bits_to_f64(inp.q_pe[b]).reshape(ql, H, wl.d_rope)[rows]
        pos = S - ql + np.asarray(rows, dtype=np.int64)
        out[n], lse[n] = prefill_explicit(qn, qp, C, Kr, w_uk, w_uv, pos, wl.softmax_scale,
                                          wl.rope_base, heads)
    return {"out": out, "lse": lse}
