"""Expected results of one decode step, from the seeded inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Takes the dict made by ``workloads.make_inputs`` and computes, in fp64:
the query (projection or given), the cache contents after the step's append
(prefilled tokens plus the new token at position prefill_len), and the
attention output for the requested sequences, and the output projection with
its FP8 pack. FP8 caches are quantised with this package's own codec.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import mfa

DEFAULT_EPS = 1e-6


def query(inp: Dict, eps: float = DEFAULT_EPS) -> np.ndarray:
    """q [B][H][d] in fp64."""
    w = inp["workload"]
    if w.has_qproj:
        a = w.act_dtype
        return mfa.query_projection(
            mfa.stored_to_f64(inp["x"], a), mfa.stored_to_f64(inp["w_qdown"], a),
            np.asarray(inp["g"], dtype=np.float64), mfa.stored_to_f64(inp["w_qup"], a),
            w.heads, w.head_dim, eps)
    return mfa.stored_to_f64(inp["q"], w.act_dtype).reshape(w.batch, w.heads, w.head_dim)


def new_token(inp: Dict):
    """Stored values (bf16 bits or fp32) of every sequence's new token, [B][d]
    each: given (``k_new``, ``v_new``), or, with ``w_kv``, the K/V projection
    of x rounded once to the activation dtype."""
    if "w_kv" not in inp:
        return inp["k_new"], inp["v_new"]
    if "_projected_token" in inp:                 # computed once per input dict
        return inp["_projected_token"]
    w = inp["workload"]
    a = w.act_dtype
    k, v = mfa.kv_projection(mfa.stored_to_f64(inp["x"], a), mfa.stored_to_f64(inp["w_kv"], a),
                             w.head_dim)
    if a == "f32":
        res = (k.astype(np.float32), v.astype(np.float32))
    else:
        res = (mfa.f64_to_bf16_bits(k), mfa.f64_to_bf16_bits(v))
    inp["_projected_token"] = res
    return res


def sequence_tokens(inp: Dict, b: int):
    """Stored logical K and V rows (prefill + appended token) of sequence b."""
    o = inp["ctx_offsets"]
    kn, vn = new_token(inp)
    k = np.concatenate([inp["k_ctx"][o[b]:o[b + 1]], kn[b:b + 1]])
    v = np.concatenate([inp["v_ctx"][o[b]:o[b + 1]], vn[b:b + 1]])
    return k, v


def sequence_kv_f64(inp: Dict, b: int):
    """fp64 values the attention of sequence b sees, plus (for FP8) the codes
    and scales: returns (k, v, extra) with extra = (kc, ks, vc, vs) or None."""
    w = inp["workload"]
    k, v = sequence_tokens(inp, b)
    if w.kv_dtype == "fp8":
        kf = mfa.bf16_bits_to_f64(k)
        vf = mfa.bf16_bits_to_f64(v)
        kc, ks = mfa.quantize_tokens(kf)
        vc, vs = mfa.quantize_tokens(vf)
        return (mfa.dequantize_tokens(kc, ks), mfa.dequantize_tokens(vc, vs),
                (kc, ks, vc, vs))
    return mfa.stored_to_f64(k, w.kv_dtype), mfa.stored_to_f64(v, w.kv_dtype), None


def physical_cache(inp: Dict, seqs: Sequence[int]):
    """Token-major fp64 physical caches holding the given sequences (zeros
    elsewhere), filled through the block table (or the contiguous mapping)."""
    w = inp["workload"]
    nrows = inp["num_blocks"] * mfa.BLOCK_TOKENS
    kc = np.zeros((nrows, w.head_dim))
    vc = np.zeros((nrows, w.head_dim))
    for b in seqs:
        k, v, _ = sequence_kv_f64(inp, b)
        mfa.scatter_tokens(kc, b, 0, k, inp["block_table"], inp["max_blocks_per_seq"])
        mfa.scatter_tokens(vc, b, 0, v, inp["block_table"], inp["max_blocks_per_seq"])
    return kc, vc


def decode_step(inp: Dict, seqs: Optional[Sequence[int]] = None,
                sm_scale: Optional[float] = None, eps: float = DEFAULT_EPS,
                fp8_queries: bool = False) -> Dict:
    """q for all sequences and the attention output for ``seqs``; with
    ``fp8_queries`` the attention uses q's per-(token, head) e4m3
    dequantisation."""
    w = inp["workload"]
    if seqs is None:
        seqs = list(range(w.batch))
    if sm_scale is None:
        sm_scale = mfa.default_sm_scale(w.head_dim)
    q = query(inp, eps)
    if fp8_queries:
        q = mfa.dequantize_queries(*mfa.quantize_queries(q))
    kc, vc = physical_cache(inp, seqs)
    o = mfa.decode_attention(q, kc, vc, inp["block_table"], inp["max_blocks_per_seq"],
                             inp["seq_lens"], sm_scale, seqs=seqs)
    return {"q": q, "o": o, "seqs": list(seqs)}


def expected_cache_rows(inp: Dict, seqs: Sequence[int]):
    """Stored K/V values (bf16 bits, e4m3 codes or fp32) and FP8 scales of the
    given sequences after the append, as token-major physical rows
    [num_blocks*64][d] (rows of other sequences are zero), plus the physical
    rows each sequence owns. ``oracle.layout`` turns rows into the library's
    block storage order and back."""
    w = inp["workload"]
    nrows = inp["num_blocks"] * mfa.BLOCK_TOKENS
    d = w.head_dim
    store = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[w.kv_dtype]
    krows = np.zeros((nrows, d), dtype=store)
    vrows = np.zeros((nrows, d), dtype=store)
    ks = np.zeros(nrows, dtype=np.float32)
    vs = np.zeros(nrows, dtype=np.float32)
    owned = {}
    for b in seqs:
        L = int(inp["seq_lens"][b])
        rows = mfa.physical_rows(b, L, inp["block_table"], inp["max_blocks_per_seq"])
        owned[b] = rows
        k, v = sequence_tokens(inp, b)
        if w.kv_dtype == "fp8":
            _, _, (kcodes, kscale, vcodes, vscale) = sequence_kv_f64(inp, b)
            krows[rows], vrows[rows] = kcodes, vcodes
            ks[rows], vs[rows] = kscale, vscale
        else:
            krows[rows], vrows[rows] = k, v
    res = {"k": krows, "v": vrows}
    if w.kv_dtype == "fp8":
        res["k_scale"] = ks
        res["v_scale"] = vs
    return res, owned


def decode_step_multi(inp: Dict, seqs: Optional[Sequence[int]] = None,
                      sm_scale: Optional[float] = None, fp8_queries: bool = False) -> np.ndarray:
    """Multi-token decode: the queries ``q_multi`` [B][T][H][d] of the last T
    tokens of every sequence (the cache after the step's append), causal
    among themselves (``fp8_queries``: their e4m3 dequantisation). Returns
    o [len(seqs)][T][H][d] in fp64."""
    w = inp["workload"]
    if seqs is None:
        seqs = list(range(w.batch))
    if sm_scale is None:
        sm_scale = mfa.default_sm_scale(w.head_dim)
    q = mfa.stored_to_f64(inp["q_multi"], w.act_dtype)
    if fp8_queries:
        q = mfa.dequantize_queries(*mfa.quantize_queries(q))
    kc, vc = physical_cache(inp, seqs)
    return mfa.decode_attention_multi(q, kc, vc, inp["block_table"], inp["max_blocks_per_seq"],
                                      inp["seq_lens"], sm_scale, seqs=seqs)


def output_projection(inp: Dict, o: Optional[np.ndarray] = None) -> Dict:
    """The output projection of the drawn attention output ``o_attn`` (or of
    ``o`` [B][H][d] / [B][H*d] in fp64, e.g. this module's decode_step output)
    through the drawn ``w_o``: y in fp64, its bf16 rounding, and the FP8
    attention-to-FFN pack of that rounding."""
    w = inp["workload"]
    if o is None:
        o = mfa.stored_to_f64(inp["o_attn"], w.act_dtype)
    y = mfa.output_projection(o, mfa.stored_to_f64(inp["w_o"], w.act_dtype))
    bits = mfa.f64_to_bf16_bits(y)
    codes, scales = mfa.a2f_pack(bits)
    return {"y": y, "y_bits": bits, "codes": codes, "scales": scales}
