"""The five synthetic decode workloads (shapes, value distributions, paging).

Each workload is a plain description; `workload.generate.make_inputs` turns it
into seeded arrays.  Nothing here computes any part of the attention method.

Shapes follow DeepSeek-V2-Lite and DeepSeek-V3 MLA decode (d_c = 512 latent,
d_rope = 64 decoupled RoPE width, d_nope = d_v = 128 per head), as described in
"DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%" (sheratonhq.com) §2.1 and
"LLM推理优化的新范式：从内存墙到计算墙的跨越" (zskr.cn) §2.1-§2.2
(seq 4096 / 8192 decode, batch 128 per GPU at seq 8192).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    page_size: int
    # exactly one of: explicit lengths, a uniform length, or a log-uniform range
    seq_lens: Optional[Sequence[int]] = None
    seq_len: Optional[int] = None
    seq_range: Optional[tuple] = None
    fp8: bool = False
    # new tokens per sequence scored in one pass (speculative verification of
    # multi-token-prediction drafts); they are the last q_len cached tokens
    q_len: int = 1
    rope_base: float = 10000.0
    spare_pages: int = 3
    seed: int = 0
    description: str = ""

    @property
    def d_latent(self) -> int:
        """Elements per cached token: c_kv (d_c) followed by rotated k_pe (d_rope)."""
        return self.d_c + self.d_rope

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    @property
    def max_seq_len(self) -> int:
        if self.seq_lens is not None:
            return max(self.seq_lens)
        if self.seq_len is not None:
            return self.seq_len
        return self.seq_range[1]

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


TINY = Workload(
    name="tiny", batch=2, n_heads=4, d_c=32, d_rope=16, d_nope=16, d_v=16,
    page_size=16, seq_lens=(37, 64),
    description="B=2 H=4 d_c=32 d_rope=16 d_nope=d_v=16 seq_lens=[37,64] page 16, shuffled pages")

V2LITE = Workload(
    name="v2lite", batch=16, n_heads=16, d_c=512, d_rope=64, d_nope=128, d_v=128,
    page_size=64, seq_len=4096,
    description="DeepSeek-V2-Lite-shaped decode: B=16 H=16 S=4096 page 64, bf16")

V3 = Workload(
    name="v3", batch=64, n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
    page_size=64, seq_len=8192,
    description="DeepSeek-V3-shaped decode: B=64 H=128 S=8192 page 64, bf16 latent cache, permuted pages")

RAGGED = Workload(
    name="ragged", batch=128, n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
    page_size=64, seq_range=(512, 32768),
    description="Ragged batch: B=128 H=128 S_b log-uniform in [512, 32768] page 64, bf16")

FP8LONG = Workload(
    name="fp8long", batch=4, n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
    page_size=64, seq_len=131072, fp8=True,
    description="Long context: B=4 H=128 S=131072 page 64, fp8 e4m3 cache + per-token fp32 scale")

# Multi-token query: the verification pass over q_len draft tokens per
# sequence ("deepseek.csdn.net" section 6: drafts from the multi-token-prediction
# layers verified by the main model in one parallel pass, e.g. 4 drafts;
# agent.csdn.net section 5.3: the first two or three drafts are usually kept).
V3_MTP2 = V3.with_(name="v3mtp2", q_len=2,
                   description="DeepSeek-V3-shaped verification pass: B=64 q_len=2 H=128 S=8192 page 64, bf16")

ALL = {w.name: w for w in (TINY, V2LITE, V3, RAGGED, FP8LONG, V3_MTP2)}


def get(name: str) -> Workload:
    return ALL[name]
