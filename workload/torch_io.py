"""Move generated inputs to device tensors (data movement only)."""
from __future__ import annotations

import numpy as np
import torch


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device` (no rounding)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def i32_tensor(x: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def to_device(inp, device="cuda") -> dict:
    """All arrays of a generated workload as device tensors, plus the per-token
    positions / sequence ids used to append the cache."""
    return {
        "seq_lens": i32_tensor(inp.seq_lens, device),
        "block_table": i32_tensor(inp.block_table, device),
        "q_nope": bf16_tensor(inp.q_nope, device),
        "q_pe": bf16_tensor(inp.q_pe, device),
        "q_pos": i32_tensor(inp.q_pos(), device),
        "c_kv": bf16_tensor(inp.c_kv, device),
        "k_pe": bf16_tensor(inp.k_pe, device),
        "positions": i32_tensor(inp.positions(), device),
        "seq_ids": i32_tensor(inp.seq_ids(), device),
        "w_uk": bf16_tensor(inp.w_uk, device),
        "w_uv": bf16_tensor(inp.w_uv, device),
    }


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
