"""Seeded synthetic inputs for MLA decode, shared by the tests, the benchmark and
the oracle's callers.

This module only draws random numbers and lays them out.  It holds none of the
attention method's arithmetic: no RoPE, no projection, no softmax, no fp8
quantisation.  The one numeric step here is rounding the fp32 draws to bf16
(round-to-nearest-even), which is how the bf16 *inputs* are made.

Draw order, for a fixed seed (numpy PCG64 `default_rng`):
  seq_lens (ragged only) -> page permutation -> q_nope -> q_pe -> c_kv -> k_pe
  -> W_UK -> W_UV.
Values: q_nope, q_pe, c_kv, k_pe ~ N(0, 1); W_UK, W_UV ~ N(0, 1/d_c).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .configs import Workload

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot overflow 32 bits here (max 0xFF7FFFFF + 0x8000)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    return (r >> np.uint32(16)).astype(np.uint16)


@dataclass
class DecodeInputs:
    wl: Workload
    seq_lens: np.ndarray      # int32 [B]
    cu_seqlens: np.ndarray    # int64 [B+1], token offsets into c_kv / k_pe
    block_table: np.ndarray   # int32 [B][max_pages]; -1 = unused entry
    num_pages: int            # physical pages in the pool (includes spares)
    q_nope: np.ndarray        # uint16 bf16 bits [B][H][d_nope]  ([B][q_len][H][d_nope] if q_len > 1)
    q_pe: np.ndarray          # uint16 bf16 bits [B][H][d_rope]  (likewise; un-rotated)
    c_kv: np.ndarray          # uint16 bf16 bits [T][d_c]          (sequence-major)
    k_pe: np.ndarray          # uint16 bf16 bits [T][d_rope]       (un-rotated)
    w_uk: np.ndarray          # uint16 bf16 bits [H][d_c][d_nope]
    w_uv: np.ndarray          # uint16 bf16 bits [H][d_c][d_v]

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def positions(self) -> np.ndarray:
        """Position of every cached token inside its sequence (int32 [T])."""
        return np.concatenate([np.arange(s, dtype=np.int32) for s in self.seq_lens]) \
            if len(self.seq_lens) else np.zeros(0, np.int32)

    def seq_ids(self) -> np.ndarray:
        """Owning sequence of every cached token (int32 [T])."""
        return np.repeat(np.arange(len(self.seq_lens), dtype=np.int32), self.seq_lens)

    def q_pos(self) -> np.ndarray:
        """Query position: the current token is the last cached one (int32 [B]);
        with q_len > 1 new tokens, they are the last q_len cached ones
        (int32 [B][q_len], position seq_len - q_len + i)."""
        ql = self.wl.q_len
        if ql == 1:
            return (self.seq_lens - 1).astype(np.int32)
        return (self.seq_lens[:, None] - ql + np.arange(ql)[None, :]).astype(np.int32)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    # Works through one reused chunk buffer: fresh large allocations are slow on
    # some hosts, and the draw sequence is the same as one big call.
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = min(n, 1 << 22)
    v = np.empty(chunk, dtype=np.float32)
    u = v.view(np.uint32)
    r = np.empty(chunk, dtype=np.uint32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        m = e - s
        rng.standard_normal(out=v[:m], dtype=np.float32)
        if sigma != 1.0:
            np.multiply(v[:m], np.float32(sigma), out=v[:m])
        # round to nearest even on the top 16 bits (finite values only)
        np.right_shift(u[:m], np.uint32(16), out=r[:m])
        np.bitwise_and(r[:m], np.uint32(1), out=r[:m])
        np.add(r[:m], np.uint32(0x7FFF), out=r[:m])
        np.add(r[:m], u[:m], out=r[:m])
        np.right_shift(r[:m], np.uint32(16), out=r[:m])
        out[s:e] = r[:m]
    return out.reshape(shape)


def make_seq_lens(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    if wl.seq_lens is not None:
        return np.asarray(wl.seq_lens, dtype=np.int32)
    if wl.seq_len is not None:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    lo, hi = wl.seq_range
    u = rng.uniform(math.log(lo), math.log(hi), size=wl.batch)
    return np.clip(np.round(np.exp(u)), lo, hi).astype(np.int32)


def make_inputs(wl: Workload, seed: int | None = None) -> DecodeInputs:
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, H = wl.batch, wl.n_heads
    seq_lens = make_seq_lens(wl, rng)
    assert len(seq_lens) == B
    ps = wl.page_size
    pages_per_seq = (seq_lens.astype(np.int64) + ps - 1) // ps
    used = int(pages_per_seq.sum())
    num_pages = used + wl.spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, int(pages_per_seq.max()) if B else 1)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seq_lens.astype(np.int64))
    T = int(cu[-1])
    qs = (B, H) if wl.q_len == 1 else (B, wl.q_len, H)
    q_nope = _normal_bf16(rng, qs + (wl.d_nope,), 1.0)
    q_pe = _normal_bf16(rng, qs + (wl.d_rope,), 1.0)
    c_kv = _normal_bf16(rng, (T, wl.d_c), 1.0)
    k_pe = _normal_bf16(rng, (T, wl.d_rope), 1.0)
    sw = 1.0 / math.sqrt(wl.d_c)
    w_uk = _normal_bf16(rng, (H, wl.d_c, wl.d_nope), sw)
    w_uv = _normal_bf16(rng, (H, wl.d_c, wl.d_v), sw)
    return DecodeInputs(wl=wl, seq_lens=seq_lens, cu_seqlens=cu, block_table=bt,
                        num_pages=num_pages, q_nope=q_nope, q_pe=q_pe, c_kv=c_kv,
                        k_pe=k_pe, w_uk=w_uk, w_uv=w_uv)


def unused_slots(inp: DecodeInputs):
    """(page, slot) pairs of the pool that no sequence owns: spare pages and the
    tail slots of each sequence's last page.  Tests fill them with NaN."""
    ps = inp.wl.page_size
    owned = set()
    slots = []
    for b in range(len(inp.seq_lens)):
        S = int(inp.seq_lens[b])
        n = (S + ps - 1) // ps
        for i in range(n):
            p = int(inp.block_table[b, i])
            owned.add(p)
            if i == n - 1:
                for s in range(S - i * ps, ps):
                    slots.append((p, s))
    spare = [p for p in range(inp.num_pages) if p not in owned]
    return spare, slots


@dataclass
class ProjectionInputs:
    """Hidden states of new tokens and the down-projection weight (nn.Linear
    layout: rows are the d_c latent outputs, then the d_rope RoPE-key outputs)."""
    h: np.ndarray             # uint16 bf16 bits [T][d_model]
    w_down: np.ndarray        # uint16 bf16 bits [d_c + d_rope][d_model]


def make_projection_inputs(n_tokens: int, d_model: int, d_latent: int, seed: int = 0) -> ProjectionInputs:
    """h ~ N(0, 1), w_down ~ N(0, 1/d_model) (so the projected values have unit
    variance), drawn in that order from numpy PCG64 `default_rng(seed)`."""
    rng = np.random.default_rng(seed)
    h = _normal_bf16(rng, (n_tokens, d_model), 1.0)
    w = _normal_bf16(rng, (d_latent, d_model), 1.0 / math.sqrt(d_model))
    return ProjectionInputs(h=h, w_down=w)
