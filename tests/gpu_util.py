"""Helpers for the GPU parity tests: set up a workload on the device through
libmfa's own calls, run the step, bring results back as fp64 numpy."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads

# bf16 / FP8 tolerances of the parity contract; fp32 self-check bound
REL_L2_BF16 = 5e-3
MAX_ABS_BF16 = 2e-2
REL_L2_F32 = 1e-5


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def max_abs(got, want) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))


def check_bf16_bars(got, want, what: str) -> None:
    """The bf16 / FP8-KV parity bars: rel-L2 <= 5e-3 and max abs <= 2e-2."""
    r, m = rel_l2(got, want), max_abs(got, want)
    say(f"{what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= REL_L2_BF16 and m <= MAX_ABS_BF16, (what, r, m)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def setup(inp, device="cuda", num_splits=None, chunk_tokens=None, zero_cache=True,
          poison=False, out_dtype=None):
    """Upload inputs, allocate + prefill the cache, build the decode step.
    ``poison``: fill every byte of the cache (and FP8 scales) with 0xFF
    before the prefill, so slots no token was written to hold NaNs."""
    import decode_attention_02_amd as mfa
    from decode_attention_02_amd.step import DecodeStep, prefill

    w = inp["workload"]
    T = workloads.to_torch(inp, device)
    cache = mfa.KVCache(inp["num_blocks"], w.head_dim, w.kv_dtype, inp["max_blocks_per_seq"],
                        block_table=T["block_table"], device=device, zero=zero_cache)
    if poison:
        for t in (cache.k, cache.v, cache.k_scale, cache.v_scale):
            if t is not None:
                t.view(torch.uint8).fill_(0xFF)
    prefill(cache, T["k_ctx"], T["v_ctx"], inp["ctx_offsets"], inp["prefill_lens"])
    act = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
    if num_splits is None and w.num_splits is not None:
        num_splits = w.num_splits
    step = DecodeStep(cache, w.batch, w.heads, int(inp["seq_lens"].max()), hidden=w.hidden,
                      q_rank=w.q_rank, act_dtype=act, num_splits=num_splits,
                      chunk_tokens=chunk_tokens, seq_lens_host=inp["seq_lens"],
                      out_dtype=out_dtype)
    return T, cache, step


def run(T, step):
    """One decode step; returns (q, out) as torch tensors on the device."""
    w = T["workload"]
    if w.has_qproj:
        out = step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], x=T["x"],
                   weights=(T["w_qdown"], T["g"], T["w_qup"]))
        q = step.q
    else:
        q = T["q"]
        out = step(T["k_new"], T["v_new"], T["prefill_lens"], T["seq_lens"], q=q)
    torch.cuda.synchronize()
    return q, out


def cache_rows(cache):
    """Stored K and V of a GPU cache as token-major rows [num_blocks*64][d]
    (bf16 as uint16 bits, FP8 as uint8 codes, fp32 as float32), undoing the
    library's block storage order with the oracle's restatement of it."""
    from oracle import layout
    dt = cache.dtype
    d = cache.head_dim

    def raw(t):
        t = t.detach().cpu()
        if dt == "bf16":
            return t.view(torch.int16).numpy().view(np.uint16).reshape(t.shape[0], -1)
        return t.numpy().reshape(t.shape[0], -1)
    k = layout.k_rows_from_blocks(raw(cache.k), d, dt)
    v = layout.v_rows_from_blocks(raw(cache.v), d, dt)
    return k, v
