"""Plain fp64 definition of the MFA decode step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``). numpy only.

Every step below is the textbook definition of what it names, computed in
float64 from the exactly upcast stored inputs. No blocking, no fusion, no
online softmax: online softmax, split-KV and paging are exact reorganisations
of the same sum, so the plain definition is the oracle for all of them.

Source: "Step-3 is Large yet Affordable: Model-system Co-design for
Cost-effective Decoding" (summary page), §2 Step-3 Model Card (MFA: low-rank
factorisation in the QK circuit, many heads, small KV cache), §5
Model-System Co-design (one 8-bit KV head shared by all heads: arithmetic
intensity 128; KV quantisation), §7 Implementation and Results (attention
instances own the KV caches).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import e4m3

BLOCK_TOKENS = 64
FP8_MAX = 448.0


# --------------------------------------------------------------------------
# stored values -> fp64
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored array: ``f32`` floats or ``bf16`` bits."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# query path: down-projection -> RMSNorm -> up-projection into H heads
# --------------------------------------------------------------------------
def rmsnorm(c: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with gain: c / sqrt(mean(c^2) + eps) * g, over the last axis.

    The pages name no normalisation for the query latent; RMSNorm with a gain
    and eps inside the root is the reading taken here.
    """
    c = np.asarray(c, dtype=np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    return c / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def query_projection(x, w_qdown, g, w_qup, heads: int, head_dim: int,
                     eps: float = 1e-6) -> np.ndarray:
    """Low-rank query path of MFA (§2 Step-3 Model Card, QK-circuit factorisation).

    x [B][Dm], w_qdown [r][Dm], g [r], w_qup [H*d][r] (weights as [out][in],
    y = x W^T). Returns q [B][H][d]; head h is output columns h*d .. h*d+d-1.
    """
    x = np.asarray(x, dtype=np.float64)
    c = x @ np.asarray(w_qdown, dtype=np.float64).T          # [B][r]
    n = rmsnorm(c, g, eps)                                    # [B][r]
    q = n @ np.asarray(w_qup, dtype=np.float64).T             # [B][H*d]
    return q.reshape(x.shape[0], heads, head_dim)


def kv_projection(x, w_kv, head_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """The new token's key and value: k = x W_k^T, v = x W_v^T.

    x [B][Dm]; w_kv [2d][Dm] is W_k stacked over W_v (weights as [out][in]).
    The attention instance computes them from the layer input and appends
    them to the cache it owns (§7 Implementation and Results); the pages give
    no positional rotation, so none is applied. Returns (k, v), each [B][d].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_kv, dtype=np.float64)
    kv = x @ w.T                                              # [B][2d]
    return kv[:, :head_dim], kv[:, head_dim:2 * head_dim]


def output_projection(o, w_o) -> np.ndarray:
    """Attention output projection y = o W_o^T.

    o [B][H][d] or [B][H*d] (heads concatenated, head h in columns
    h*d .. h*d+d-1); w_o [Dm][H*d] as [out][in]. Returns y [B][Dm]. The
    attention instance hands y on to the FFN instances (§7 Implementation and
    Results); the pages give no bias, so none is added.
    """
    o = np.asarray(o, dtype=np.float64)
    o = o.reshape(o.shape[0], -1)
    return o @ np.asarray(w_o, dtype=np.float64).T


def a2f_pack(y_bf16_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 hand-off of bf16 hidden states from attention to FFN.

    §7 (Implementation and Results) of the summary page has attention send
    FP8 tokens with their scales to the FFN side; the StepMesh page's traffic
    model counts one byte per hidden element. Reading taken here: the bf16
    row is quantised per token exactly as the FP8 KV cache is (one fp32 scale
    amax/448 per row, RNE e4m3 codes of the correctly rounded fp32
    quotient). Returns (codes uint8 [B][Dm], scales float32 [B]).
    """
    return quantize_tokens(bf16_bits_to_f64(np.asarray(y_bf16_bits, dtype=np.uint16)))


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp64 values to bfloat16 bit patterns.

    bfloat16 keeps 8 significant bits and fp32's exponent range: each value
    is rounded once, directly from fp64, to a multiple of 2^(e-8) (e its
    binary exponent, 2^(e-1) <= |a| < 2^e; subnormal step 2^-133), ties to
    even. Values must be finite and below the bf16 overflow threshold.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(a / step) * step                              # exact: fits 8 bits
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# attention of H heads against one shared K/V head
# --------------------------------------------------------------------------
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      sm_scale: float) -> np.ndarray:
    """o[h] = softmax_t(q[h].k[t] * sm_scale) . v  for q [H][d], k/v [L][d].

    Every head attends to the same K and V (the single shared KV head). L = 0
    gives zeros (nothing to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    s = (q @ k.T) * sm_scale                                  # [H][L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def physical_rows(b: int, length: int, block_table: Optional[np.ndarray],
                  max_blocks_per_seq: int) -> np.ndarray:
    """Physical token rows of sequence b's logical tokens 0..length-1.

    Logical token t lives in logical block t // 64 at offset t % 64; the block
    table maps logical block j of sequence b to a physical block id. Without a
    table the cache is contiguous: logical block j of sequence b is physical
    block b * max_blocks_per_seq + j.
    """
    t = np.arange(length, dtype=np.int64)
    j = t // BLOCK_TOKENS
    if block_table is None:
        blk = b * max_blocks_per_seq + j
    else:
        blk = np.asarray(block_table, dtype=np.int64)[b, j]
    return blk * BLOCK_TOKENS + t % BLOCK_TOKENS


def scatter_tokens(cache_rows: np.ndarray, b: int, start: int, rows: np.ndarray,
                   block_table: Optional[np.ndarray], max_blocks_per_seq: int) -> None:
    """Write ``rows`` [n][...] as logical tokens start..start+n-1 of sequence b
    into a token-major physical cache ``cache_rows`` [num_blocks*64][...]."""
    n = rows.shape[0]
    phys = physical_rows(b, start + n, block_table, max_blocks_per_seq)[start:]
    cache_rows[phys] = rows


def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     block_table: Optional[np.ndarray], max_blocks_per_seq: int,
                     seq_lens: Sequence[int], sm_scale: float,
                     seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """Decode attention over a (paged or contiguous) token-major cache.

    q [B][H][d]; k_cache, v_cache [num_blocks*64][d] fp64 token rows. Returns
    o [len(seqs)][H][d] for the sequences in ``seqs`` (default: all).
    """
    q = np.asarray(q, dtype=np.float64)
    if seqs is None:
        seqs = range(q.shape[0])
    out = []
    for b in seqs:
        rows = physical_rows(b, int(seq_lens[b]), block_table, max_blocks_per_seq)
        out.append(softmax_attention(q[b], k_cache[rows], v_cache[rows], sm_scale))
    return np.stack(out)


def decode_attention_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                           block_table: Optional[np.ndarray], max_blocks_per_seq: int,
                           seq_lens: Sequence[int], sm_scale: float,
                           seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """Several new tokens per sequence, attending causally.

    q [B][T][H][d]: the queries of the last T tokens of every sequence (the
    tokens decoded together in one step, as multi-token prediction does, §5
    of the summary page). Query j (0-based) of sequence b sees the sequence's
    first seq_lens[b] - (T - 1 - j) tokens: everything before the new tokens
    plus new tokens 0..j. Returns o [len(seqs)][T][H][d].
    """
    q = np.asarray(q, dtype=np.float64)
    T = q.shape[1]
    if seqs is None:
        seqs = range(q.shape[0])
    out = []
    for b in seqs:
        per_token = []
        for j in range(T):
            n = max(int(seq_lens[b]) - (T - 1 - j), 0)
            rows = physical_rows(b, n, block_table, max_blocks_per_seq)
            per_token.append(softmax_attention(q[b, j], k_cache[rows], v_cache[rows], sm_scale))
        out.append(np.stack(per_token))
    return np.stack(out)


# --------------------------------------------------------------------------
# split-KV partials and their log-sum-exp combine
# --------------------------------------------------------------------------
def split_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                   chunk: int, num_splits: int) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Per-chunk (o, m, l) of one sequence: chunk j covers tokens
    [j*chunk, min((j+1)*chunk, L)). o is the unnormalised sum
    sum_t exp(s_t - m) v_t, m the chunk's max scaled logit (natural-log units),
    l = sum_t exp(s_t - m). An empty chunk gives (0, -inf, 0)."""
    q = np.asarray(q, dtype=np.float64)
    L = k.shape[0]
    parts = []
    for j in range(num_splits):
        lo, hi = j * chunk, min((j + 1) * chunk, L)
        if hi <= lo:
            parts.append((np.zeros((q.shape[0], v.shape[1])),
                          np.full(q.shape[0], -np.inf), np.zeros(q.shape[0])))
            continue
        s = (q @ np.asarray(k[lo:hi], dtype=np.float64).T) * sm_scale
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        parts.append((p @ np.asarray(v[lo:hi], dtype=np.float64), m, p.sum(axis=1)))
    return parts


def combine(parts) -> np.ndarray:
    """Merge chunk partials (o_j, m_j, l_j) into the normalised output.

    m* = max_j m_j; weights w_j = exp(m_j - m*) (0 for empty chunks);
    o = sum_j w_j o_j / sum_j w_j l_j. All chunks empty gives zeros.
    """
    o_list = [np.asarray(p[0], dtype=np.float64) for p in parts]
    m = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])    # [S][H]
    l = np.stack([np.asarray(p[2], dtype=np.float64) for p in parts])    # [S][H]
    m_star = m.max(axis=0)
    H = m.shape[1]
    out = np.zeros_like(o_list[0])
    for h in range(H):
        if not np.isfinite(m_star[h]):
            continue
        w = np.where(np.isfinite(m[:, h]), np.exp(np.where(np.isfinite(m[:, h]),
                                                           m[:, h] - m_star[h], 0.0)), 0.0)
        num = sum(w[j] * o_list[j][h] for j in range(len(o_list)))
        out[h] = num / np.dot(w, l[:, h])
    return out


# --------------------------------------------------------------------------
# FP8 e4m3 KV with one fp32 scale per token (per K and per V)
# --------------------------------------------------------------------------
def quantize_tokens(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token e4m3 quantisation of rows x [n][d] (values exact in fp32).

    Per row: amax = max_i |x_i|; s = fp32(amax / 448) (one correctly rounded
    fp32 division; s = 1 when amax = 0); code_i = RNE_e4m3(fp32(x_i / s)).
    |x_i / s| <= 448 * (1 + 2^-23) < 464, the midpoint above 448, so no code
    saturates. Returns (codes uint8 [n][d], scales float32 [n]).

    Reading taken here of the summary page's "8-bit KV" (§5): OCP e4m3 codes,
    one scale per token for K and one for V, scale = amax / 448.
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    y = (x32 / s[:, None]).astype(np.float32)
    return e4m3.encode_rne(y), s


def quantize_queries(q: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 queries: each (token, head) row of q [..][H][d] quantised on its
    own with the KV cache's per-token codec (``quantize_tokens``). Reading
    taken here of the summary page's FP8 attention (§7): one scale per head
    row, so a head's logits keep its own range. Returns (codes [..][H][d],
    scales float32 [..][H])."""
    q = np.asarray(q, dtype=np.float64)
    codes, s = quantize_tokens(q.reshape(-1, q.shape[-1]))
    return codes.reshape(q.shape), s.reshape(q.shape[:-1])


def dequantize_queries(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(code) * scale of every (token, head) row, exact in fp64."""
    d = codes.shape[-1]
    return dequantize_tokens(codes.reshape(-1, d), np.asarray(scales).reshape(-1)).reshape(
        codes.shape)


def dequantize_tokens(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(code) * scale, exact in fp64."""
    return e4m3.decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def default_sm_scale(head_dim: int) -> float:
    """1/sqrt(d): the usual scaled dot-product factor."""
    return 1.0 / math.sqrt(head_dim)
