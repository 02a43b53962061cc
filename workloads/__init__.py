"""Seeded synthetic inputs for the MFA decode step.

This module draws random numbers and casts them to their storage dtypes. It
holds none of the method's arithmetic: no projection, normalisation, softmax,
quantisation or cache layout lives here. Both the oracle (``oracle/``) and the
GPU path (tests, ``bench.py``) take their inputs from it, and that is all the
two sides share.

Shapes follow the Step-3 MFA attention as summarised on the page "Step-3 is
Large yet Affordable: Model-system Co-design for Cost-effective Decoding"
(§2 Model Card: one attention per block with a low-rank QK circuit; §5
Model-System Co-design: arithmetic intensity 128 with 8-bit KV, effective rank
16,384, i.e. 64 query heads of width 256 sharing one KV head).

Conventions
-----------
* numpy PCG64 ``default_rng(seed)``; values drawn in float32 and cast
  round-to-nearest-even to the storage dtype (bf16 is returned as its uint16
  bit pattern, fp32 as float32).
* Draw order: per-sequence lengths, then x, W_qdown, g, W_qup (or q when the
  workload has no query projection), then prefilled K, prefilled V, k_new,
  v_new, then the block permutation.
* "context" is the attended length. The last token of every sequence is the
  one written by the decode step's KV append; the cache is prefilled with the
  tokens before it. The paged mixed-length workload draws the pre-append
  length and attends over one more.
* Physical cache blocks hold 64 tokens. Paged workloads assign a random
  permutation of all blocks in (sequence, logical block) order; unused table
  entries are -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_TOKENS = 64
# Step-3's hidden width, for workloads that draw q directly: 128 tokens of it
# are 896 KiB in FP8 on the StepMesh page's attention-to-FFN traffic model.
STEP3_HIDDEN = 7168


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload."""

    name: str
    batch: int
    hidden: Optional[int]        # None: q is drawn directly (no query projection)
    q_rank: Optional[int]
    heads: int
    head_dim: int
    kv_dtype: str                # "f32" | "bf16" | "fp8"
    act_dtype: str               # dtype of x, weights, q: "f32" | "bf16"
    context: Optional[int]       # fixed attended length (None: drawn)
    context_range: Optional[tuple] = None  # inclusive pre-append length range
    paged: bool = False
    num_splits: Optional[int] = None       # fixed split count, None: library plan

    @property
    def has_qproj(self) -> bool:
        return self.hidden is not None


# The five workloads. Index = position in the project's list of decode shapes.
WORKLOADS = {
    1: Workload("tiny-fp32", batch=2, hidden=256, q_rank=128, heads=4, head_dim=64,
                kv_dtype="f32", act_dtype="f32", context=128),
    2: Workload("step3-bf16-4k", batch=32, hidden=7168, q_rank=2048, heads=64,
                head_dim=256, kv_dtype="bf16", act_dtype="bf16", context=4096),
    3: Workload("paged-bf16-mixed", batch=128, hidden=None, q_rank=None, heads=64,
                head_dim=256, kv_dtype="bf16", act_dtype="bf16", context=None,
                context_range=(1024, 8192), paged=True),
    4: Workload("paged-fp8-32k", batch=16, hidden=None, q_rank=None, heads=64,
                head_dim=256, kv_dtype="fp8", act_dtype="bf16", context=32768,
                paged=True),
    5: Workload("split32-bf16-64k", batch=4, hidden=7168, q_rank=2048, heads=64,
                head_dim=256, kv_dtype="bf16", act_dtype="bf16", context=65536,
                num_splits=32),
}


def default_seed(index: int) -> int:
    """Seed of workload ``index``: the tiny case fixes 0, the others use index-1."""
    return index - 1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 draws to the storage dtype. fp8 caches take bf16 inputs."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype in ("bf16", "fp8"):
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def make_inputs(index: int, seed: Optional[int] = None, batch: Optional[int] = None,
                context: Optional[int] = None, workload: Optional[Workload] = None,
                prefill_lens=None, kv_proj: bool = False, q_len: int = 1,
                out_proj: bool = False):
    """Draw the inputs of one decode step of workload ``index``.

    ``batch`` / ``context`` shrink the workload (for tests that need a small
    instance of the same structure); ``workload`` replaces it entirely;
    ``prefill_lens`` fixes the pre-append lengths (no length draw).

    Returns a dict of numpy arrays in storage form (see module docstring):
    ``x, w_qdown, g, w_qup`` or ``q``; ``k_ctx, v_ctx`` ([sum prefill][d],
    sequence-major) with ``ctx_offsets`` [B+1]; ``k_new, v_new`` [B][d];
    ``prefill_lens`` and ``seq_lens`` [B] int32; ``block_table`` [B][max_blocks]
    int32 or None; ``num_blocks``, ``max_blocks_per_seq``; plus the workload.
    ``kv_proj`` (query-path workloads only) also draws ``w_kv`` [2d][hidden]
    (W_k over W_v, N(0, 1/hidden)) after everything else, so the other
    arrays are the same with and without it; the new token is then the K/V
    projection of x and ``k_new`` / ``v_new`` are not its values.
    ``q_len`` > 1 (workloads that draw q) also draws ``q_multi``
    [B][q_len][H][d], the queries of the last q_len tokens of every sequence
    (multi-token decode), after everything else.
    ``out_proj`` also draws, after all of the above, ``o_attn`` [B][H*d]
    (an attention output, N(0, 1)) and ``w_o`` [hidden][H*d] (N(0, 1/(H*d))),
    hidden being the workload's (Step-3's 7168 when it has no query path).
    """
    w = workload if workload is not None else WORKLOADS[index]
    if batch is not None or context is not None:
        w = dataclasses.replace(
            w, batch=batch if batch is not None else w.batch,
            context=context if (context is not None and w.context is not None) else w.context)
    if seed is None:
        seed = default_seed(index)
    rng = np.random.default_rng(seed)
    B, H, d = w.batch, w.heads, w.head_dim
    act = w.act_dtype
    kvin = "f32" if w.kv_dtype == "f32" else "bf16"

    # 1. lengths
    if prefill_lens is not None:
        prefill = np.asarray(prefill_lens, dtype=np.int64)
        w = dataclasses.replace(w, batch=len(prefill))
        B = w.batch
    elif w.context_range is not None:
        lo, hi = w.context_range
        if context is not None:           # shrunk instance keeps the spread, scaled
            lo, hi = max(1, context // 8), context
        prefill = rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    else:
        prefill = np.full(B, w.context - 1, dtype=np.int64)
    seq_lens = prefill + 1

    out = {"workload": w, "seed": seed}
    # 2. query path
    if w.has_qproj:
        Dm, r = w.hidden, w.q_rank
        out["x"] = _store(rng.standard_normal((B, Dm), dtype=np.float32), act)
        out["w_qdown"] = _store(rng.standard_normal((r, Dm), dtype=np.float32)
                                / np.float32(math.sqrt(Dm)), act)
        out["g"] = (np.float32(1.0) + np.float32(0.1)
                    * rng.standard_normal(r, dtype=np.float32)).astype(np.float32)
        out["w_qup"] = _store(rng.standard_normal((H * d, r), dtype=np.float32)
                              / np.float32(math.sqrt(r)), act)
    else:
        out["q"] = _store(rng.standard_normal((B, H, d), dtype=np.float32), act)

    # 3. cache contents
    total = int(prefill.sum())
    out["k_ctx"] = _store(rng.standard_normal((total, d), dtype=np.float32), kvin)
    out["v_ctx"] = _store(rng.standard_normal((total, d), dtype=np.float32), kvin)
    out["k_new"] = _store(rng.standard_normal((B, d), dtype=np.float32), kvin)
    out["v_new"] = _store(rng.standard_normal((B, d), dtype=np.float32), kvin)
    offs = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(prefill, out=offs[1:])
    out["ctx_offsets"] = offs
    out["prefill_lens"] = prefill.astype(np.int32)
    out["seq_lens"] = seq_lens.astype(np.int32)

    # 4. blocks
    nblk = (seq_lens + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    max_blocks = int(nblk.max())
    if w.paged:
        num_blocks = int(nblk.sum())
        perm = rng.permutation(num_blocks).astype(np.int32)
        bt = np.full((B, max_blocks), -1, dtype=np.int32)
        pos = 0
        for b in range(B):
            n = int(nblk[b])
            bt[b, :n] = perm[pos:pos + n]
            pos += n
        out["block_table"] = bt
        out["num_blocks"] = num_blocks
    else:
        out["block_table"] = None
        out["num_blocks"] = B * max_blocks
    out["max_blocks_per_seq"] = max_blocks

    # 5. K/V projection weights (drawn last)
    if kv_proj:
        if not w.has_qproj:
            raise ValueError("the K/V projection needs a query-path workload (x)")
        out["w_kv"] = _store(rng.standard_normal((2 * d, w.hidden), dtype=np.float32)
                             / np.float32(math.sqrt(w.hidden)), act)

    # 6. queries of several new tokens per sequence (drawn last)
    if q_len > 1:
        if w.has_qproj:
            raise ValueError("multi-token queries are drawn for workloads without a query path")
        out["q_multi"] = _store(rng.standard_normal((B, q_len, H, d), dtype=np.float32), act)

    # 7. attention output and the output projection weight (drawn last)
    if out_proj:
        hid = w.hidden if w.has_qproj else STEP3_HIDDEN
        out["o_attn"] = _store(rng.standard_normal((B, H * d), dtype=np.float32), act)
        out["w_o"] = _store(rng.standard_normal((hid, H * d), dtype=np.float32)
                            / np.float32(math.sqrt(H * d)), act)
    return out


def to_torch(inp, device="cuda"):
    """Copy the drawn arrays to ``device`` as torch tensors (bf16 bits are
    reinterpreted as torch.bfloat16, fp32 stays float32, int32 stays int32).
    Pure data movement."""
    import torch

    w = inp["workload"]

    def t(a, dt):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
            torch.bfloat16).to(device)

    kvin = "f32" if w.kv_dtype == "f32" else "bf16"
    out = {"workload": w}
    if w.has_qproj:
        for k in ("x", "w_qdown", "w_qup"):
            out[k] = t(inp[k], w.act_dtype)
        if "w_kv" in inp:
            out["w_kv"] = t(inp["w_kv"], w.act_dtype)
        out["g"] = torch.from_numpy(inp["g"]).to(device)
    else:
        out["q"] = t(inp["q"], w.act_dtype)
        if "q_multi" in inp:
            out["q_multi"] = t(inp["q_multi"], w.act_dtype)
    for k in ("o_attn", "w_o"):
        if k in inp:
            out[k] = t(inp[k], w.act_dtype)
    for k in ("k_ctx", "v_ctx", "k_new", "v_new"):
        out[k] = t(inp[k], kvin)
    out["ctx_offsets"] = inp["ctx_offsets"]
    out["prefill_lens"] = torch.from_numpy(inp["prefill_lens"]).to(device)
    out["seq_lens"] = torch.from_numpy(inp["seq_lens"]).to(device)
    out["block_table"] = (torch.from_numpy(inp["block_table"]).to(device)
                          if inp["block_table"] is not None else None)
    for k in ("num_blocks", "max_blocks_per_seq"):
        out[k] = inp[k]
    out["prefill_host"] = inp["prefill_lens"]
    out["seq_lens_host"] = inp["seq_lens"]
    return out
