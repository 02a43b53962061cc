"""Bytes and flop of the MFA decode step, per unit of work.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The summary page "Step-3 is Large yet Affordable" states the cost model in
§4 (Cost Analysis for LLM Decoding): attention cost is the larger of its
computation and its KV-memory access, plus the linear projections. §5
(Model-System Co-design) gives MFA's arithmetic intensity as 128 with an 8-bit
KV cache, and its effective rank as 16,384.

Per cached token of one sequence, with H query heads of width d sharing one
KV head of width d stored in b bytes per element:
  bytes = 2 * d * b          (one K row and one V row)
  flop  = 4 * H * d          (q.k for H heads: 2Hd; p.v for H heads: 2Hd)
so the intensity is 2H/b.
"""
from __future__ import annotations


def kv_bytes_per_token(head_dim: int, elem_bytes: float, scale_bytes: int = 0) -> float:
    """K row + V row, plus per-token scale bytes for K and for V."""
    return 2 * head_dim * elem_bytes + 2 * scale_bytes


def attn_flop_per_token(heads: int, head_dim: int) -> int:
    """Multiply-adds of q.k and p.v over all heads, counted as 2 flop each."""
    return 2 * heads * head_dim + 2 * heads * head_dim


def arithmetic_intensity(heads: int, head_dim: int, elem_bytes: float,
                         scale_bytes: int = 0) -> float:
    return attn_flop_per_token(heads, head_dim) / kv_bytes_per_token(
        head_dim, elem_bytes, scale_bytes)


def effective_rank(heads: int, head_dim: int) -> int:
    """Total query width H*d (the page's "effective rank" reading)."""
    return heads * head_dim


def qproj_weight_bytes(hidden: int, q_rank: int, heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    return (hidden * q_rank + q_rank * heads * head_dim) * elem_bytes


def qproj_flop(batch: int, hidden: int, q_rank: int, heads: int, head_dim: int) -> int:
    return 2 * batch * (hidden * q_rank + q_rank * heads * head_dim)


def hidden_payload_bytes(tokens: int, hidden: int, elem_bytes: int, scale_bytes: int = 0) -> int:
    """Bytes of hidden states sent one way between attention and FFN
    instances: tokens x hidden elements, plus a per-token scale if any (the
    StepMesh page's traffic model: FP8 from attention to FFN, BF16 back)."""
    return tokens * (hidden * elem_bytes + scale_bytes)
