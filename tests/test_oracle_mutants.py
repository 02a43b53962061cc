"""Planted mistakes in copies of the oracle must each fail at least one pin.

The mistakes are planted here, on the CPU, in functions that wrap or replace
oracle functions; the oracle itself is untouched.
"""
import math
import types

import numpy as np
import pytest

import pins
from oracle import e4m3, mfa


def _mut(**over):
    O = pins.real_oracle()
    d = dict(vars(O))
    d.update(over)
    return types.SimpleNamespace(**d)


def _attn_no_scale(q, k, v, sm_scale):
    return mfa.softmax_attention(q, k, v, 1.0)


def _attn_heads_axis(q, k, v, sm_scale):
    s = (np.asarray(q) @ np.asarray(k).T) * sm_scale
    p = np.exp(s - s.max(axis=0, keepdims=True))
    return (p / p.sum(axis=0, keepdims=True)) @ v


def _attn_drop_last(q, k, v, sm_scale):
    if len(k) > 1:
        k, v = k[:-1], v[:-1]
    return mfa.softmax_attention(q, k, v, sm_scale)


def _attn_k_as_v(q, k, v, sm_scale):
    if k.shape == v.shape:
        v = k
    return mfa.softmax_attention(q, k, v, sm_scale)


def _rows_wrong_offset(b, length, bt, mb):
    t = np.arange(length)
    j = t // 64
    blk = (b * mb + j) if bt is None else np.asarray(bt)[b, j]
    return blk * 64 + (t % 64 + 1) % 64


def _rows_contig_swapped(b, length, bt, mb):
    if bt is not None:
        return mfa.physical_rows(b, length, bt, mb)
    t = np.arange(length)
    return (t // 64 * 4 + b) * 64 + t % 64


def _combine_no_rescale(parts):
    o = sum(np.asarray(p[0]) for p in parts)
    l = sum(np.asarray(p[2]) for p in parts)
    return o / l[:, None]


def _combine_drop_last(parts):
    return mfa.combine(parts[:-1]) if len(parts) > 1 else mfa.combine(parts)


def _rms_no_gain(c, g, eps):
    return mfa.rmsnorm(c, np.ones_like(np.asarray(g, dtype=float)), eps)


def _rms_sum(c, g, eps):
    c = np.asarray(c, dtype=float)
    return c / np.sqrt(np.sum(c * c, axis=-1, keepdims=True) + eps) * g


def _qproj_head_transposed(x, wd, g, wu, H, d, eps):
    q = mfa.query_projection(x, wd, g, wu, H, d, eps)
    return q.reshape(q.shape[0], d, H).transpose(0, 2, 1).copy()


def _decode_bias8(codes):
    return e4m3.decode(codes) / 2.0


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(x)
    idx = np.abs(a[:, None] - pos[None, :])
    best = np.argmin(idx[:, ::-1], axis=1)
    code = (0x7E - best).astype(np.uint8)          # ties resolved to the larger value
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), 448.0)
    code = (np.searchsorted(pos, a, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _quant_wrong_max(x):
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = np.where(amax == 0, 1.0, amax / np.float32(240.0)).astype(np.float32)
    return e4m3.encode_rne((x32 / s[:, None]).astype(np.float32)), s


def _quant_scale_by_reciprocal(x):
    # s = amax * fl(1/448): two roundings instead of one correctly rounded division
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = (amax * (np.float32(1.0) / np.float32(448.0))).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    return e4m3.encode_rne((x32 / s[:, None]).astype(np.float32)), s


def _a2f_scale_by_reciprocal(bits):
    return _quant_scale_by_reciprocal(mfa.bf16_bits_to_f64(bits))


def _qq_scale_by_reciprocal(q):
    q = np.asarray(q, float)
    c, sc = _quant_scale_by_reciprocal(q.reshape(-1, q.shape[-1]))
    return c.reshape(q.shape), sc.reshape(q.shape[:-1])


def _ai_qk_only(H, d, b, sb=0):
    return 2 * H * d / (2 * d * b + 2 * sb)


def _k_blocks_gc_swapped(rows, dt):
    from oracle import layout
    if dt != "bf16":
        return layout.k_blocks(rows, dt)
    x = rows.reshape(-1, 4, 16, rows.shape[1] // 32, 4, 8).transpose(0, 1, 3, 2, 4, 5)
    return np.ascontiguousarray(x).reshape(x.shape[0], -1)


def _multi_not_causal(q, kc, vc, bt, mb, lens, sc, seqs=None):
    # every query token sees all seq_lens[b] tokens
    T = np.asarray(q).shape[1]
    return np.stack([mfa.decode_attention(np.asarray(q)[:, j], kc, vc, bt, mb, lens, sc, seqs)
                     for j in range(T)], axis=1)


def _multi_off_by_one(q, kc, vc, bt, mb, lens, sc, seqs=None):
    # query j sees one token fewer than it should
    T = np.asarray(q).shape[1]
    return np.stack([mfa.decode_attention(np.asarray(q)[:, j], kc, vc, bt, mb,
                                          [max(L - (T - j), 0) for L in lens], sc, seqs)
                     for j in range(T)], axis=1)


def _kv_swapped(x, w, d):
    k, v = mfa.kv_projection(x, w, d)
    return v, k


def _oproj_heads_reversed(o, w):
    o = np.asarray(o, float)
    if o.ndim == 3:
        o = o[:, ::-1]
    return mfa.output_projection(o, w)


def _oproj_weight_not_transposed(o, w):
    o = np.asarray(o, float).reshape(len(o), -1)
    w = np.asarray(w, float)
    return o @ w if w.shape[0] == o.shape[1] else o @ w.T[:, ::-1]


def _a2f_signed_max(bits):
    y = mfa.bf16_bits_to_f64(bits)
    amax = np.max(y, axis=1)                   # forgets the absolute value
    s = np.where(amax == 0, 1.0, amax / 448.0).astype(np.float32)
    return e4m3.encode_rne((y / s[:, None]).astype(np.float32)), s


def _a2f_e4m3_max_240(bits):
    y = mfa.bf16_bits_to_f64(bits)
    amax = np.max(np.abs(y), axis=1)
    s = np.where(amax == 0, 1.0, amax / 240.0).astype(np.float32)
    return e4m3.encode_rne((y / s[:, None]).astype(np.float32)), s


def _a2f_no_scale(bits):
    y = mfa.bf16_bits_to_f64(bits)
    return e4m3.encode_rne(y), np.ones(len(y), np.float32)


def _payload_with_scales(tokens, hidden, elem_bytes, scale_bytes=0):
    return tokens * (hidden * elem_bytes + 4)


def _qq_one_scale_per_token(q):
    q = np.asarray(q, float)
    flat = q.reshape(-1, q.shape[-2] * q.shape[-1])          # all heads of a token together
    c, sc = mfa.quantize_tokens(flat)
    return c.reshape(q.shape), np.repeat(sc, q.shape[-2]).reshape(q.shape[:-1])


def _qq_truncates(q):
    q = np.asarray(q, float)
    d = q.shape[-1]
    rows = q.reshape(-1, d).astype(np.float32)
    amax = np.max(np.abs(rows), axis=1)
    sc = np.where(amax == 0, 1.0, amax / 448.0).astype(np.float32)
    y = rows / sc[:, None]
    vals = e4m3.DECODE_TABLE[:0x7F]
    idx = np.searchsorted(vals, np.abs(y), side="right") - 1     # round toward zero
    c = idx.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return c.reshape(q.shape), sc.reshape(q.shape[:-1])


def _kv_rows_offset(x, w, d):
    # the weight rows read one row off (W_k / W_v halves misaligned)
    kv = np.asarray(x, float) @ np.roll(np.asarray(w, float), 1, axis=0).T
    return kv[:, :d], kv[:, d:2 * d]


def _bf16_truncate(a):
    a32 = np.asarray(a, np.float64).astype(np.float32)
    return (a32.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_ties_away(a):
    a = np.asarray(a, np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.sign(a) * np.floor(np.abs(a) / step + 0.5) * step
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


MUTANTS = {
    "multi_token_not_causal": dict(decode_attention_multi=_multi_not_causal),
    "multi_token_off_by_one": dict(decode_attention_multi=_multi_off_by_one),
    "kv_projection_k_v_swapped": dict(kv_projection=_kv_swapped),
    "kv_projection_rows_offset": dict(kv_projection=_kv_rows_offset),
    "output_projection_heads_reversed": dict(output_projection=_oproj_heads_reversed),
    "output_projection_weight_not_transposed": dict(output_projection=_oproj_weight_not_transposed),
    "a2f_pack_signed_max": dict(a2f_pack=_a2f_signed_max),
    "a2f_pack_e4m3_max_240": dict(a2f_pack=_a2f_e4m3_max_240),
    "a2f_pack_no_scale": dict(a2f_pack=_a2f_no_scale),
    "a2f_payload_counts_scales": dict(hidden_payload_bytes=_payload_with_scales),
    "fp8_queries_one_scale_per_token": dict(quantize_queries=_qq_one_scale_per_token),
    "fp8_queries_truncate": dict(quantize_queries=_qq_truncates),
    "bf16_round_truncates": dict(f64_to_bf16_bits=_bf16_truncate),
    "bf16_round_ties_away": dict(f64_to_bf16_bits=_bf16_ties_away),
    "attention_missing_scale": dict(softmax_attention=_attn_no_scale),
    "attention_softmax_over_heads": dict(softmax_attention=_attn_heads_axis),
    "attention_drops_last_token": dict(softmax_attention=_attn_drop_last),
    "attention_uses_k_for_v": dict(softmax_attention=_attn_k_as_v),
    "gather_offset_off_by_one": dict(physical_rows=_rows_wrong_offset),
    "gather_contiguous_swapped": dict(physical_rows=_rows_contig_swapped),
    "combine_without_rescale": dict(combine=_combine_no_rescale),
    "combine_drops_last_split": dict(combine=_combine_drop_last),
    "rmsnorm_drops_gain": dict(rmsnorm=_rms_no_gain),
    "rmsnorm_sum_not_mean": dict(rmsnorm=_rms_sum),
    "qproj_heads_transposed": dict(query_projection=_qproj_head_transposed),
    "e4m3_wrong_bias": dict(e4m3_decode=_decode_bias8),
    "e4m3_ties_away": dict(e4m3_encode=_encode_ties_away),
    "e4m3_truncates": dict(e4m3_encode=_encode_truncate),
    "quant_wrong_max": dict(quantize_tokens=_quant_wrong_max),
    "quant_scale_by_reciprocal": dict(quantize_tokens=_quant_scale_by_reciprocal),
    "a2f_pack_scale_by_reciprocal": dict(a2f_pack=_a2f_scale_by_reciprocal),
    "fp8_queries_scale_by_reciprocal": dict(quantize_queries=_qq_scale_by_reciprocal),
    "cost_counts_qk_only": dict(arithmetic_intensity=_ai_qk_only),
    "layout_lane_order_swapped": dict(k_blocks=_k_blocks_gc_swapped),
}


def _wire(name, O):
    """Mutated helpers must reach the checks that compose them."""
    if name.startswith("gather"):
        pr = O.physical_rows

        def dec(q, kc, vc, bt, mb, lens, sc, seqs=None):
            seqs = range(len(q)) if seqs is None else seqs
            return np.stack([mfa.softmax_attention(q[b], kc[pr(b, lens[b], bt, mb)],
                                                   vc[pr(b, lens[b], bt, mb)], sc) for b in seqs])

        def scat(cache, b, start, rows, bt, mb):
            phys = pr(b, start + rows.shape[0], bt, mb)[start:]
            cache[phys] = rows
        O.decode_attention, O.scatter_tokens = dec, scat
    if name == "rmsnorm_drops_gain" or name == "rmsnorm_sum_not_mean":
        rn = O.rmsnorm

        def qp(x, wd, g, wu, H, d, eps):
            n = rn(np.asarray(x, float) @ np.asarray(wd, float).T, g, eps)
            return (n @ np.asarray(wu, float).T).reshape(len(x), H, d)
        O.query_projection = qp
    if name == "e4m3_wrong_bias":
        O.dequantize_tokens = lambda c, s: _decode_bias8(c) * np.asarray(s, float)[:, None]
    return O


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    O = _wire(name, _mut(**MUTANTS[name]))
    fails = pins.run_all(O)
    assert fails, f"planted mistake {name} passed every pin"
