"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` takes a namespace of oracle functions and returns a list of
failure messages (empty = pinned). ``test_oracle.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies with a planted mistake
and expects at least one failure, which shows that the pins would catch it.

What pins what:
* attention  -- pure-Python brute force; one token returns V exactly; constant
  K returns the mean of V; two tokens follow the logistic closed form; a
  dominant logit returns that token's V; a common shift of K along q leaves
  the output unchanged; zero scale gives the mean of V; reordering tokens
  changes nothing beyond rounding.
* gather     -- a hand-worked block-table example; permuted physical blocks
  give a bit-identical output.
* split / combine -- any split count (with empty chunks) reproduces the
  unsplit brute-force result; two hand-built partials merge by closed form.
* rmsnorm / query projection -- output RMS equals 1 before the gain; scale
  invariance; constant input gives the gain; identity down-projection reduces
  to W_up x / rms(x); pure-Python brute force; head h owns columns h*d..h*d+d-1.
* multi-token decode -- each query token equals single-token decode at its
  causal length; a later new token is invisible to earlier queries and
  visible to its own; pure-Python brute force.
* K/V projection -- block-identity weights give x's halves exactly; row
  mapping of W_k / W_v; pure-Python brute force.
* output projection -- identity weight returns o; head h reaches only its
  own column block; [B][H][d] and [B][H*d] agree; pure-Python brute force.
* A2F pack -- hand-worked rows (scale 1 and scale 2, negative amax, zero
  row) coded bit for bit; the amax element codes to +-448; error within half
  an e4m3 step times the scale; the page's 896 KiB / 1.75 MiB payloads.
* bf16 rounding -- anchor values including exact ties (to even) and values
  next to them; torch's RNE cast of fp32 values; the half-ulp error bound.
* e4m3 -- torch's float8_e4m3fn decode of all 256 codes; anchor values of the
  OCP format; round trip of every finite value; midpoints round to even;
  torch's RNE cast on random values.
* quantisation -- the amax element encodes to +-448; error within half an
  e4m3 step times the scale; zero rows; sign kept.
* FP8 queries -- every (token, head) row on its own: scaling one head moves
  only that head's scale and leaves its codes; rows already on the e4m3 grid
  with amax 448 round-trip exactly; attention with such queries equals
  attention with the originals; the amax element of each head codes to 448.
* cost -- the page's intensity 128 at 8-bit KV and effective rank 16,384.
* block layout -- hand-worked element positions of the documented storage
  order, a bijection, and the inverse undoing the forward map.
"""
from __future__ import annotations

import json
import math
import os
import types

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def real_oracle():
    from oracle import brute, cost, e4m3, layout, mfa
    return types.SimpleNamespace(
        softmax_attention=mfa.softmax_attention,
        physical_rows=mfa.physical_rows,
        decode_attention=mfa.decode_attention,
        decode_attention_multi=mfa.decode_attention_multi,
        scatter_tokens=mfa.scatter_tokens,
        split_partials=mfa.split_partials,
        combine=mfa.combine,
        rmsnorm=mfa.rmsnorm,
        query_projection=mfa.query_projection,
        kv_projection=mfa.kv_projection,
        output_projection=mfa.output_projection,
        a2f_pack=mfa.a2f_pack,
        hidden_payload_bytes=cost.hidden_payload_bytes,
        f64_to_bf16_bits=mfa.f64_to_bf16_bits,
        quantize_tokens=mfa.quantize_tokens,
        dequantize_tokens=mfa.dequantize_tokens,
        quantize_queries=mfa.quantize_queries,
        dequantize_queries=mfa.dequantize_queries,
        e4m3_decode=e4m3.decode,
        e4m3_encode=e4m3.encode_rne,
        arithmetic_intensity=cost.arithmetic_intensity,
        effective_rank=cost.effective_rank,
        kv_bytes_per_token=cost.kv_bytes_per_token,
        k_blocks=layout.k_blocks,
        v_blocks=layout.v_blocks,
        k_rows_from_blocks=layout.k_rows_from_blocks,
        v_rows_from_blocks=layout.v_rows_from_blocks,
        pack_weight=layout.pack_weight,
        brute=brute,
    )


def _close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and np.all(np.abs(a - b) <= tol * (1.0 + np.abs(b)))


# ---------------------------------------------------------------- attention
def check_attention(O):
    fails = []
    rng = np.random.default_rng(1234)
    # brute force on tiny random cases
    for trial in range(12):
        H = int(rng.integers(1, 5))
        d = int(rng.integers(1, 9))
        L = int(rng.integers(1, 17))
        dv = int(rng.integers(1, 9))
        q = rng.standard_normal((H, d)) * 2
        k = rng.standard_normal((L, d))
        v = rng.standard_normal((L, dv))
        sc = float(rng.uniform(0.1, 1.5))
        got = O.softmax_attention(q, k, v, sc)
        want = O.brute.attention(q.tolist(), k.tolist(), v.tolist(), sc)
        if not _close(got, want, 1e-12):
            fails.append(f"brute force mismatch H={H} d={d} L={L}")
            break
    # one token: exactly V for every head
    q = rng.standard_normal((4, 8)); k = rng.standard_normal((1, 8)); v = rng.standard_normal((1, 8))
    got = O.softmax_attention(q, k, v, 0.35)
    if not np.array_equal(got, np.repeat(v, 4, axis=0)):
        fails.append("L=1 does not return V exactly")
    # constant K: mean of V
    k = np.repeat(rng.standard_normal((1, 8)), 9, axis=0)
    v = rng.standard_normal((9, 5))
    got = O.softmax_attention(q, k, v, 0.7)
    if not _close(got, np.repeat(v.mean(axis=0, keepdims=True), 4, axis=0), 1e-13):
        fails.append("constant K does not give mean of V")
    # two tokens: o = sigma(delta) v0 + (1 - sigma(delta)) v1
    q = rng.standard_normal((3, 6)); k = rng.standard_normal((2, 6)); v = rng.standard_normal((2, 4))
    sc = 0.5
    got = O.softmax_attention(q, k, v, sc)
    for h in range(3):
        delta = sc * (q[h] @ k[0] - q[h] @ k[1])
        a = 1.0 / (1.0 + math.exp(-delta))
        if not _close(got[h], a * v[0] + (1 - a) * v[1], 1e-13):
            fails.append("two-token logistic closed form fails")
            break
    # dominant logit: output equals that token's V
    d = 8
    k = np.zeros((5, d)); k[3, 0] = 1.0
    q = np.zeros((2, d)); q[:, 0] = 2000.0
    v = rng.standard_normal((5, 3))
    got = O.softmax_attention(q, k, v, 1.0)
    if not np.array_equal(got, np.repeat(v[3:4], 2, axis=0)):
        fails.append("dominant logit does not select its V row")
    # shifting every key by the same vector: logits of a head shift uniformly
    q = rng.standard_normal((3, 6)); k = rng.standard_normal((7, 6)); v = rng.standard_normal((7, 6))
    shift = rng.standard_normal(6)
    a = O.softmax_attention(q, k, v, 0.4)
    b = O.softmax_attention(q, k + shift, v, 0.4)
    if not _close(a, b, 1e-12):
        fails.append("common key shift changes the output")
    # zero scale: uniform weights, mean of V
    got = O.softmax_attention(q, k, v, 0.0)
    if not _close(got, np.repeat(v.mean(axis=0, keepdims=True), 3, axis=0), 1e-13):
        fails.append("zero scale does not give mean of V")
    # token order does not matter
    perm = rng.permutation(7)
    b = O.softmax_attention(q, k[perm], v[perm], 0.4)
    if not _close(a, b, 1e-12):
        fails.append("token permutation changes the output")
    return fails


# ---------------------------------------------------------------- gather
def check_gather(O):
    fails = []
    with open(os.path.join(GOLDEN, "gather_example.json")) as f:
        ex = json.load(f)
    bt = np.array(ex["block_table"], dtype=np.int32)
    for c in ex["cases"]:
        rows = O.physical_rows(c["seq"], c["length"], bt, ex["max_blocks_per_seq"])
        if "rows" in c and rows.tolist() != c["rows"]:
            fails.append(f"gather example rows {c}")
        if "tokens" in c and rows[c["tokens"]].tolist() != c["rows_at_tokens"]:
            fails.append(f"gather example tokens {c}")
    cg = ex["contiguous"]
    for c in cg["cases"]:
        rows = O.physical_rows(c["seq"], c["length"], None, cg["max_blocks_per_seq"])
        if rows[c["tokens"]].tolist() != c["rows_at_tokens"]:
            fails.append(f"contiguous example {c}")
    # permuted physical blocks: identical output
    rng = np.random.default_rng(7)
    B, H, d, L = 3, 4, 8, 150
    nblk = 3
    q = rng.standard_normal((B, H, d))
    kl = rng.standard_normal((B, L, d))
    vl = rng.standard_normal((B, L, d))
    outs = []
    for trial in range(2):
        perm = rng.permutation(B * nblk).astype(np.int32)
        bt = perm.reshape(B, nblk)
        kc = np.zeros((B * nblk * 64, d)); vc = np.zeros_like(kc)
        for b in range(B):
            O.scatter_tokens(kc, b, 0, kl[b], bt, nblk)
            O.scatter_tokens(vc, b, 0, vl[b], bt, nblk)
        outs.append(O.decode_attention(q, kc, vc, bt, nblk, [L] * B, 0.3))
    if not np.array_equal(outs[0], outs[1]):
        fails.append("permuted physical blocks change the output")
    direct = np.stack([O.brute.attention(q[b].tolist(), kl[b].tolist(), vl[b].tolist(), 0.3)
                       for b in range(B)])
    if not _close(outs[0], direct, 1e-12):
        fails.append("paged attention differs from brute force on logical rows")
    return fails


# ---------------------------------------------------------------- split / combine
def check_combine(O):
    fails = []
    rng = np.random.default_rng(99)
    H, d, L = 3, 5, 37
    q = rng.standard_normal((H, d)) * 1.5
    k = rng.standard_normal((L, d)); v = rng.standard_normal((L, d))
    want = np.array(O.brute.attention(q.tolist(), k.tolist(), v.tolist(), 0.6))
    for S, chunk in ((1, 64), (2, 19), (3, 13), (32, 2), (32, 64)):
        parts = O.split_partials(q, k, v, 0.6, chunk, S)
        got = O.combine(parts)
        if not _close(got, want, 1e-12):
            fails.append(f"split S={S} chunk={chunk} differs from unsplit")
    # hand-built: two partials of one head
    o1, m1, l1 = np.array([[2.0, 4.0]]), np.array([1.0]), np.array([2.0])
    o2, m2, l2 = np.array([[1.0, -1.0]]), np.array([3.0]), np.array([1.0])
    e = math.exp(-2.0)
    want = (e * o1[0] + o2[0]) / (e * 2.0 + 1.0)
    empty = (np.zeros((1, 2)), np.array([-np.inf]), np.zeros(1))
    got = O.combine([(o1, m1, l1), empty, (o2, m2, l2)])
    if not _close(got[0], want, 1e-14):
        fails.append("two-partial closed form fails")
    return fails


# ---------------------------------------------------------------- rmsnorm / qproj
def check_qproj(O):
    fails = []
    rng = np.random.default_rng(5)
    c = rng.standard_normal((3, 16)) * 3
    n1 = O.rmsnorm(c, np.ones(16), 0.0)
    if not _close(np.sqrt(np.mean(n1 * n1, axis=1)), np.ones(3), 1e-14):
        fails.append("RMS of normalised rows is not 1")
    g = 1 + 0.1 * rng.standard_normal(16)
    if not _close(O.rmsnorm(c * 7.5, g, 0.0), O.rmsnorm(c, g, 0.0), 1e-14):
        fails.append("rmsnorm not scale invariant")
    if not _close(O.rmsnorm(np.full((1, 16), -2.5), g, 0.0)[0], -g, 1e-14):
        fails.append("constant row does not give -g")
    # identity down-projection, unit gain: q = W_up x / rms(x)
    r, H, d = 8, 2, 3
    x = rng.standard_normal((2, r))
    wu = rng.standard_normal((H * d, r))
    q = O.query_projection(x, np.eye(r), np.ones(r), wu, H, d, 0.0)
    for b in range(2):
        want = wu @ (x[b] / (np.linalg.norm(x[b]) / math.sqrt(r)))
        if not _close(q[b].reshape(-1), want, 1e-13):
            fails.append("identity down-projection closed form fails")
            break
    # brute force with real shapes (tiny) and eps
    Dm, r, H, d = 6, 4, 2, 3
    x = rng.standard_normal((2, Dm)); wd = rng.standard_normal((r, Dm))
    g = 1 + 0.1 * rng.standard_normal(r); wu = rng.standard_normal((H * d, r))
    got = O.query_projection(x, wd, g, wu, H, d, 1e-3)
    want = np.array(O.brute.query_projection(x.tolist(), wd.tolist(), g.tolist(), wu.tolist(),
                                             H, d, 1e-3))
    if not _close(got, want, 1e-12):
        fails.append("query projection differs from brute force")
    # head mapping: W_up row h*d+j feeds head h, dim j
    wu = np.zeros((H * d, r)); wu[1 * d + 2, 0] = 1.0
    got = O.query_projection(x, wd, g, wu, H, d, 0.0)
    nz = np.argwhere(np.abs(got) > 0)
    if not (len(nz) > 0 and np.all(nz[:, 1] == 1) and np.all(nz[:, 2] == 2)):
        fails.append("head mapping of W_up rows is wrong")
    return fails


# ---------------------------------------------------------------- multi-token decode
def check_multi_token(O):
    fails = []
    rng = np.random.default_rng(13)
    H, d, T, mb = 2, 3, 3, 2
    lens = [5, 70, 2]                        # pre-existing tokens + the T new ones
    nb = 3 * mb
    kc = rng.standard_normal((nb * 64, d)); vc = rng.standard_normal((nb * 64, d))
    bt = np.arange(nb, dtype=np.int32).reshape(3, mb)[:, ::-1].copy()   # permuted blocks
    q = rng.standard_normal((3, T, H, d))
    got = O.decode_attention_multi(q, kc, vc, bt, mb, lens, 0.5)
    # one query token at a time is single-token decode with the causal length
    for j in range(T):
        lj = [max(L - (T - 1 - j), 0) for L in lens]
        want = O.decode_attention(q[:, j], kc, vc, bt, mb, lj, 0.5)
        if not _close(got[:, j], want, 1e-13):
            fails.append(f"query token {j} differs from single-token decode at its length")
    # causality: changing the last new token changes only the last query's output
    last = [O.physical_rows(b, lens[b], bt, mb)[-1] for b in range(3)]
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[last] += 5.0; vc2[last] -= 3.0
    got2 = O.decode_attention_multi(q, kc2, vc2, bt, mb, lens, 0.5)
    if not _close(got2[:, :T - 1], got[:, :T - 1], 1e-13):
        fails.append("earlier query tokens see a later new token")
    if _close(got2[:, T - 1], got[:, T - 1], 1e-6):
        fails.append("the last query token does not see itself")
    # brute force on logical rows
    for b in range(3):
        rows = O.physical_rows(b, lens[b], bt, mb)
        for j in range(T):
            n = lens[b] - (T - 1 - j)
            if n <= 0:                       # fewer tokens than queries: nothing to attend
                if np.any(got[b, j] != 0.0):
                    fails.append(f"query token {j} of a too-short sequence is not zero")
                continue
            for h in range(H):
                want = O.brute.attention(q[b, j, h:h + 1].tolist(), kc[rows[:n]].tolist(),
                                         vc[rows[:n]].tolist(), 0.5)
                if not _close(got[b, j, h], np.array(want)[0], 1e-12):
                    fails.append(f"brute force differs at b={b} j={j} h={h}")
                    return fails
    return fails


# ---------------------------------------------------------------- K/V projection
def check_kv_projection(O):
    fails = []
    rng = np.random.default_rng(11)
    d = 3
    # W_k = [I | 0], W_v = [0 | 2I] on Dm = 2d: k = x[:, :d], v = 2 x[:, d:]
    x = rng.standard_normal((4, 2 * d))
    w = np.zeros((2 * d, 2 * d))
    w[:d, :d] = np.eye(d)
    w[d:, d:] = 2.0 * np.eye(d)
    k, v = O.kv_projection(x, w, d)
    if not (np.array_equal(k, x[:, :d]) and np.array_equal(v, 2.0 * x[:, d:])):
        fails.append("block-identity K/V projection closed form fails")
    # row j of w_kv feeds k[:, j]; row d + j feeds v[:, j]
    w = np.zeros((2 * d, 5)); w[1, 4] = 1.0; w[d + 2, 0] = -1.0
    x = rng.standard_normal((2, 5))
    k, v = O.kv_projection(x, w, d)
    want_k = np.zeros((2, d)); want_k[:, 1] = x[:, 4]
    want_v = np.zeros((2, d)); want_v[:, 2] = -x[:, 0]
    if not (np.array_equal(k, want_k) and np.array_equal(v, want_v)):
        fails.append("K/V projection row mapping is wrong")
    # pure-Python brute force
    x = rng.standard_normal((3, 7)); w = rng.standard_normal((2 * d, 7))
    k, v = O.kv_projection(x, w, d)
    bk, bv = O.brute.kv_projection(x.tolist(), w.tolist(), d)
    if not (_close(k, np.array(bk), 1e-13) and _close(v, np.array(bv), 1e-13)):
        fails.append("K/V projection differs from brute force")
    return fails


# ---------------------------------------------------------------- output projection
def check_output_projection(O):
    fails = []
    rng = np.random.default_rng(21)
    H, d = 3, 4
    o = rng.standard_normal((2, H, d))
    # identity weight (Dm = H*d): y is o with heads concatenated
    if not np.array_equal(O.output_projection(o, np.eye(H * d)), o.reshape(2, H * d)):
        fails.append("identity output projection does not return o")
    # only head 1's block of W_o set: y depends on head 1 alone
    w = np.zeros((5, H * d)); w[:, d:2 * d] = rng.standard_normal((5, d))
    o2 = o.copy(); o2[:, 0] += 7.0; o2[:, 2] -= 3.0
    y1, y2 = O.output_projection(o, w), O.output_projection(o2, w)
    if not (np.array_equal(y1, y2) and _close(y1, o[:, 1] @ w[:, d:2 * d].T, 1e-14)):
        fails.append("head h does not map to columns h*d .. h*d+d-1 of W_o")
    w = rng.standard_normal((5, H * d))
    if not np.array_equal(O.output_projection(o, w), O.output_projection(o.reshape(2, -1), w)):
        fails.append("[B][H][d] and [B][H*d] inputs differ")
    want = O.brute.output_projection(o.reshape(2, -1).tolist(), w.tolist())
    if not _close(O.output_projection(o, w), np.array(want), 1e-13):
        fails.append("output projection differs from brute force")
    return fails


def _bf16_bits(vals):
    """bf16 bit patterns of values that bf16 holds exactly (checked)."""
    a = np.asarray(vals, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), a)
    return bits


# ------------------------------------------------------- FP8 scale rounding
# The codec's scale is ONE correctly rounded fp32 division amax / 448 (the
# reading of the Step-3 summary page's 8-bit KV, §5 Model-System Co-design).
# The helpers below round exact rationals to fp32 on their own (no numpy
# float arithmetic), so they check the oracle's division from outside it.
def _f32_rne_exact(q: "Fraction") -> "Fraction":
    """Nearest fp32 value of a rational in the normal range, ties to even."""
    from fractions import Fraction
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def _f32_bits(v) -> int:
    return int(np.array([float(v)], dtype=np.float32).view(np.uint32)[0])


# A worked row (bf16 bits), derived by hand with exact rationals:
#   amax = 1.015625 = 65/64; 65/64/448 = 65/28672 lies between the fp32 values
#   0x3B149249 and 0x3B14924A and is nearer the first, which is the scale.
#   The reciprocal route amax * fl(1/448) gives 0x3B14924A instead.
#   0x3782 = 0x1.04p-16 = amax * 2^-16: its quotient rounds to exactly
#   448 * 2^-16 = 3.5 * 2^-9, the midpoint between the subnormal codes 3 and
#   4, which ties to the even code 4 (3 with the reciprocal scale's quotient,
#   just below it). 0.25 / s = 110.3 -> 112 (0x6E); 0.9375 / s = 413.5 -> 416
#   (0xFD); 0.0078125 / s = 3.446 -> 3.5 (0x46); -0.5078125 / s = -224 (0xF6).
FP8_WORKED_ROW_BITS = [0x3F82, 0xBF02, 0x3782, 0xB782, 0x0000, 0x3E80, 0xBF70, 0x3C00]
FP8_WORKED_SCALE_BITS = 0x3B149249
FP8_WORKED_CODES = [0x7E, 0xF6, 0x04, 0x84, 0x00, 0x6E, 0xFD, 0x46]


def _worked_row_f64():
    return (np.asarray(FP8_WORKED_ROW_BITS, np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_worked_fp8(codes, scale_bits, what):
    """Failure messages if a coded worked row differs from the literals."""
    fails = []
    if int(scale_bits) != FP8_WORKED_SCALE_BITS:
        fails.append(f"{what}: worked-row scale bits {int(scale_bits):#010x} != "
                     f"{FP8_WORKED_SCALE_BITS:#010x} (amax/448 not one correctly rounded division)")
    if [int(c) for c in codes] != FP8_WORKED_CODES:
        fails.append(f"{what}: worked-row codes {[hex(int(c)) for c in codes]}")
    return fails


def _check_scales_exact(amax_f32, scales, what):
    """Every scale equals the exactly rounded amax / 448 (1 for amax 0)."""
    from fractions import Fraction
    for a, s in zip(np.asarray(amax_f32, np.float32).tolist(), np.asarray(scales, np.float32).tolist()):
        want = 1.0 if a == 0 else float(_f32_rne_exact(Fraction(a) / 448))
        if _f32_bits(s) != _f32_bits(want):
            return [f"{what}: scale of amax {a!r} is {s!r}, the rounded quotient is {want!r}"]
    return []


def _bf16_rne_bits(a32):
    """bf16 bits of fp32 values, round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def check_a2f_pack(O):
    fails = []
    # worked rows: 448 -> s = 1, codes are the values' own e4m3 codes
    # (448 = 0x7E, -224 = -1.75*2^7 -> 0xF6, 1 -> 0x38, 0.5 -> 0x30, 0 -> 0x00);
    # amax 896 (negative) -> s = 2; a zero row -> s = 1, all codes 0
    rows = _bf16_bits([[448.0, -224.0, 1.0, 0.0, 0.5, 0.0, 0.0, 0.0],
                       [-896.0, 1.0, 2.0, 448.0, -0.0, 0.0, 0.0, 0.0],
                       [0.0] * 8])
    codes, s = O.a2f_pack(rows)
    want = [[0x7E, 0xF6, 0x38, 0x00, 0x30, 0, 0, 0],
            [0xFE, 0x30, 0x38, 0x76, 0x80, 0, 0, 0],
            [0] * 8]
    if not (np.array_equal(codes, np.array(want, dtype=np.uint8))
            and np.array_equal(s, np.array([1.0, 2.0, 1.0], dtype=np.float32))):
        fails.append(f"worked A2F rows: codes {codes.tolist()}, scales {s.tolist()}")
    # random rows: amax element codes to +-448, error within half a step
    rng = np.random.default_rng(22)
    y = rng.standard_normal((16, 512)) * rng.uniform(1e-3, 40, size=(16, 1))
    bits = O.f64_to_bf16_bits(y)
    yb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, s = O.a2f_pack(bits)
    j = np.argmax(np.abs(yb), axis=1)
    if not np.all((codes[np.arange(16), j] & 0x7F) == 0x7E):
        fails.append("amax element of an A2F row not coded as 448")
    deq = O.dequantize_tokens(codes, s)
    r = np.abs(deq / s[:, None].astype(np.float64))
    step = np.where(r < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 3))
    if not np.all(np.abs(deq - yb) / s[:, None] <= step / 2 * (1 + 1e-6) + 1e-30):
        fails.append("A2F pack error beyond half a step of the bf16 values")
    fails += _check_scales_exact(np.max(np.abs(yb), axis=1), s, "A2F pack")
    wc, ws = O.a2f_pack(np.asarray([FP8_WORKED_ROW_BITS], np.uint16))
    fails += _check_worked_fp8(wc[0], _f32_bits(ws[0]), "A2F pack")
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = {e["id"]: e["value"] for e in json.load(f)["figures"]}
    if O.hidden_payload_bytes(128, 7168, 1) != figs["a2f_bytes_batch128"]:
        fails.append("FP8 attention-to-FFN payload != page figure")
    if O.hidden_payload_bytes(128, 7168, 2) != figs["f2a_bytes_batch128"]:
        fails.append("BF16 FFN-to-attention payload != page figure")
    return fails


def check_bf16_round(O):
    import torch
    fails = []
    anchors = {1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000, 3.140625: 0x4049,
               1.0 + 2.0 ** -8: 0x3F80,                    # tie -> even mantissa 0
               1.0 + 3 * 2.0 ** -8: 0x3F82,                # tie -> even mantissa 2
               1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,       # just above the tie
               -(1.0 + 2.0 ** -8 - 2.0 ** -30): 0xBF80}    # just below the tie
    got = O.f64_to_bf16_bits(np.array(list(anchors)))
    for (val, want), g in zip(anchors.items(), got.tolist()):
        if g != want:
            fails.append(f"bf16 rounding of {val!r}: {g:#06x} != {want:#06x}")
    # torch's round-to-nearest-even cast on fp32 values (exact in fp64)
    rng = np.random.default_rng(12)
    a32 = (rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))).astype(np.float32)
    ref = torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(O.f64_to_bf16_bits(a32.astype(np.float64)), ref):
        fails.append("bf16 rounding differs from torch's cast")
    # error bound: half a unit in the 8th significant bit
    a = rng.standard_normal(4096) * 1e3
    r = (O.f64_to_bf16_bits(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if not np.all(np.abs(r - a) <= np.abs(a) * 2.0 ** -8):
        fails.append("bf16 rounding error above half an ulp")
    return fails


# ---------------------------------------------------------------- e4m3
def check_e4m3(O):
    import torch
    fails = []
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    if not same.all():
        fails.append(f"decode differs from torch at codes {np.flatnonzero(~same)[:8]}")
    anchors = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
               0x38: 1.0, 0x40: 2.0, 0xB8: -1.0, 0x00: 0.0, 0x07: 7 * 2.0 ** -9}
    for c, val in anchors.items():
        if O.e4m3_decode(np.array([c], dtype=np.uint8))[0] != val:
            fails.append(f"anchor code {c:#x} != {val}")
    if not (np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()):
        fails.append("NaN codes")
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    rt = O.e4m3_encode(O.e4m3_decode(finite))
    if not np.array_equal(rt, finite):
        fails.append("round trip of finite values fails")
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = O.e4m3_encode(mids)
    if not np.all(enc % 2 == 0):
        fails.append("midpoints do not round to the even code")
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1, 30, 200)]
                          + [mids, -mids]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(vals.astype(np.float64))
    # torch drops the sign of an exact zero result only for +0 inputs; compare magnitudes
    # of codes that decode to zero, and exact codes elsewhere
    dz = O.e4m3_decode(got) == 0
    if not (np.array_equal(got[~dz], ref[~dz]) and np.all((ref[dz] & 0x7F) == 0)):
        bad = np.flatnonzero((got != ref) & ~dz)[:5]
        fails.append(f"encode differs from torch RNE at {vals[bad]}")
    return fails


def check_quantize(O):
    fails = []
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((50, 256)) * rng.uniform(1e-3, 50, size=(50, 1))).astype(np.float32)
    x[7] = 0.0
    x[9, :] = -np.abs(x[9, :])
    codes, s = O.quantize_tokens(x.astype(np.float64))
    deq = O.dequantize_tokens(codes, s)
    for i in range(50):
        if i == 7:
            if not (s[i] == 1.0 and np.all(codes[i] == 0)):
                fails.append("zero row not (scale 1, code 0)")
            continue
        j = int(np.argmax(np.abs(x[i])))
        if (codes[i, j] & 0x7F) != 0x7E:
            fails.append(f"amax element of row {i} not coded as 448")
            break
    # error bound: half a step of the e4m3 grid at that magnitude, times s
    y = np.abs(deq / s[:, None].astype(np.float64))
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    err = np.abs(deq - x) / s[:, None]
    if not np.all(err <= step / 2 * (1 + 1e-6) + 1e-30):
        fails.append("quantisation error beyond half a step")
    if not np.all((codes[9] & 0x80) == 0x80):
        fails.append("sign lost for negative row")
    fails += _check_scales_exact(np.max(np.abs(x), axis=1), s, "quantize")
    # random bf16 rows: the scale is the exactly rounded quotient
    xb = (rng.standard_normal((400, 64)) * np.exp2(rng.integers(-12, 10, size=(400, 1))))
    xb = (_bf16_rne_bits(xb.astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    _, sb = O.quantize_tokens(xb.astype(np.float64))
    fails += _check_scales_exact(np.max(np.abs(xb), axis=1), sb, "quantize bf16 rows")
    wc, ws = O.quantize_tokens(_worked_row_f64()[None, :])
    fails += _check_worked_fp8(wc[0], _f32_bits(ws[0]), "quantize")
    return fails


def check_fp8_queries(O):
    fails = []
    rng = np.random.default_rng(31)
    q = rng.standard_normal((3, 2, 4, 64)).astype(np.float32).astype(np.float64)   # [B][T][H][d]
    codes, s = O.quantize_queries(q)
    if codes.shape != q.shape or s.shape != q.shape[:-1]:
        fails.append("query codes / scales shape")
        return fails
    j = np.argmax(np.abs(q), axis=-1)
    if not np.all((np.take_along_axis(codes, j[..., None], -1) & 0x7F) == 0x7E):
        fails.append("amax element of a query head not coded as 448")
    # error within half a step of the e4m3 grid, times the head's scale
    deq = O.dequantize_queries(codes, s)
    r = np.abs(deq / s[..., None].astype(np.float64))
    step = np.where(r < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 3))
    if not np.all(np.abs(deq - q) / s[..., None] <= step / 2 * (1 + 1e-6) + 1e-30):
        fails.append("query quantisation error beyond half a step")
    # one head scaled by 2^5: its scale moves by 2^5, its codes and every other head stay
    q2 = q.copy(); q2[1, 0, 2] *= 32.0
    c2, s2 = O.quantize_queries(q2)
    other = np.ones(s.shape, bool); other[1, 0, 2] = False
    if not (np.array_equal(c2, codes) and np.array_equal(s2[other], s[other])
            and s2[1, 0, 2] == np.float32(32.0) * s[1, 0, 2]):
        fails.append("query heads are not quantised independently")
    # rows already on the e4m3 grid with amax 448 (scale 1) round-trip exactly
    grid_codes = rng.integers(0, 0x7E, size=(2, 4, 64)).astype(np.uint8)
    grid_codes[..., 5] = 0x7E
    grid_codes |= (rng.integers(0, 2, size=grid_codes.shape) * 0x80).astype(np.uint8)
    qg = O.e4m3_decode(grid_codes)
    c3, s3 = O.quantize_queries(qg)
    if not (np.array_equal(s3, np.ones(s3.shape, np.float32))
            and np.array_equal(O.dequantize_queries(c3, s3), qg)):
        fails.append("queries on the e4m3 grid do not round-trip")
    # attention with such queries equals attention with the originals
    k = rng.standard_normal((40, 64)); v = rng.standard_normal((40, 64))
    qd = O.dequantize_queries(c3, s3)
    a1 = O.softmax_attention(qd[0], k, v, 0.01)
    a2 = O.softmax_attention(qg[0], k, v, 0.01)
    if not np.array_equal(a1, a2):
        fails.append("FP8-query attention differs on exactly representable queries")
    # the worked row as head 1 of a token, next to another head
    qw = np.stack([rng.standard_normal(8), _worked_row_f64()])[None]      # [1][H=2][8]
    cw, sw = O.quantize_queries(qw)
    fails += _check_worked_fp8(cw[0, 1], _f32_bits(sw[0, 1]), "FP8 queries")
    return fails


def check_cost(O):
    fails = []
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = {e["id"]: e["value"] for e in json.load(f)["figures"]}
    if O.arithmetic_intensity(64, 256, 1) != figs["mfa_ai_8bit"]:
        fails.append("intensity at 8-bit KV != page figure")
    if O.effective_rank(64, 256) != figs["mfa_effective_rank"]:
        fails.append("effective rank != page figure")
    if O.kv_bytes_per_token(256, 2) != 1024:
        fails.append("bf16 KV bytes per token")
    return fails


# Element positions inside one 64-token block with d = 256, worked by hand
# from the documented order: (kind, dtype, token, dim) -> flat element index.
LAYOUT_EXAMPLES = [
    # bf16 K: unit (17//16)*8 + 42//32 = 9, lane 16*((42%32)//8) + 17%16 = 17, j 2
    ("k", "bf16", 17, 42, (9 * 64 + 17) * 8 + 2),
    # bf16 V: unit (200//16)*2 + 37//32 = 25, lane 16*((37%32)//8) + 200%16 = 8, j 5
    ("v", "bf16", 37, 200, (25 * 64 + 8) * 8 + 5),
    # fp8 K: unit (17//16)*4 + 42//64 = 4, lane 16*((42%64)//16) + 1 = 33, j 10
    ("k", "fp8", 17, 42, (4 * 64 + 33) * 16 + 10),
    # fp8 V: unit 200//16 = 12, lane 16*(37//16) + 8 = 40, j 5
    ("v", "fp8", 37, 200, (12 * 64 + 40) * 16 + 5),
    ("k", "f32", 17, 42, 17 * 256 + 42),
    ("v", "f32", 37, 200, 200 * 64 + 37),
    ("k", "bf16", 63, 255, (31 * 64 + 63) * 8 + 7),
    ("v", "bf16", 0, 0, 0),
]


def check_layout(O):
    fails = []
    d = 256
    ids = (np.arange(64)[:, None] * d + np.arange(d)[None, :]).astype(np.int64)
    rows2 = np.concatenate([ids, ids + 64 * d])          # two blocks
    for kind, dt, t, dim, pos in LAYOUT_EXAMPLES:
        fwd = O.k_blocks if kind == "k" else O.v_blocks
        blk = fwd(ids, dt)[0]
        if blk[pos] != t * d + dim:
            fails.append(f"{kind}/{dt}: element ({t},{dim}) not at {pos}")
    for dt in ("f32", "bf16", "fp8"):
        for kind in ("k", "v"):
            fwd = O.k_blocks if kind == "k" else O.v_blocks
            inv = O.k_rows_from_blocks if kind == "k" else O.v_rows_from_blocks
            blk = fwd(rows2, dt)
            if sorted(blk[0].tolist()) != list(range(64 * d)):
                fails.append(f"{kind}/{dt}: not a permutation")
            if not np.array_equal(inv(blk, d, dt), rows2):
                fails.append(f"{kind}/{dt}: inverse does not undo the layout")
    # packed weight [32][64]: w[17][42] -> unit 1*2 + 1 = 3, lane 16*1 + 1 = 17, j 2
    wid = (np.arange(32)[:, None] * 64 + np.arange(64)[None, :]).astype(np.int64)
    pk = O.pack_weight(wid)
    if pk[(3 * 64 + 17) * 8 + 2] != 17 * 64 + 42:
        fails.append("packed weight: element (17,42) misplaced")
    if pk[(0 * 64 + 16 * 3 + 15) * 8 + 7] != 15 * 64 + 31:
        fails.append("packed weight: element (15,31) misplaced")
    if sorted(pk.tolist()) != list(range(32 * 64)):
        fails.append("packed weight: not a permutation")
    return fails


ALL_CHECKS = (check_attention, check_gather, check_combine, check_multi_token, check_qproj,
              check_kv_projection, check_output_projection, check_a2f_pack,
              check_bf16_round, check_e4m3, check_quantize, check_fp8_queries, check_cost,
              check_layout)


def run_all(O):
    fails = []
    for chk in ALL_CHECKS:
        fails.extend(f"{chk.__name__}: {m}" for m in chk(O))
    return fails
