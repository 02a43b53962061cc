"""Pure-Python brute force for tiny cases (no numpy): explicit loops, math.exp.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``). Used only to pin the
numpy oracle on inputs small enough to loop over.
"""
from __future__ import annotations

import math
from typing import List, Sequence

Vec = List[float]


def dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for x, y in zip(a, b):
        s += float(x) * float(y)
    return s


def attention(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]],
              v: Sequence[Sequence[float]], sm_scale: float) -> List[Vec]:
    """softmax(q k^T * scale) v, head by head, with an explicit max shift."""
    out = []
    for qh in q:
        logits = [dot(qh, kt) * sm_scale for kt in k]
        top = max(logits)
        e = [math.exp(s - top) for s in logits]
        z = sum(e)
        dv = len(v[0])
        out.append([sum(e[t] * float(v[t][j]) for t in range(len(v))) / z
                    for j in range(dv)])
    return out


def matvec_t(w: Sequence[Sequence[float]], x: Sequence[float]) -> Vec:
    """y = W x for W given as rows [out][in]."""
    return [dot(row, x) for row in w]


def query_projection(x: Sequence[Sequence[float]], w_qdown, g, w_qup, heads: int,
                     head_dim: int, eps: float) -> List[List[Vec]]:
    """Row by row: c = W_down x; n = c / sqrt(mean c^2 + eps) * g; q = W_up n."""
    out = []
    for xb in x:
        c = matvec_t(w_qdown, xb)
        ms = sum(ci * ci for ci in c) / len(c)
        inv = 1.0 / math.sqrt(ms + eps)
        n = [ci * inv * float(gi) for ci, gi in zip(c, g)]
        qf = matvec_t(w_qup, n)
        out.append([qf[h * head_dim:(h + 1) * head_dim] for h in range(heads)])
    return out


def kv_projection(x: Sequence[Sequence[float]], w_kv, head_dim: int):
    """Row by row: k = W_k x, v = W_v x, with W_k the first head_dim rows of
    w_kv and W_v the next head_dim rows."""
    ks, vs = [], []
    for xb in x:
        kv = matvec_t(w_kv, xb)
        ks.append(kv[:head_dim])
        vs.append(kv[head_dim:2 * head_dim])
    return ks, vs


def output_projection(o: Sequence[Sequence[float]], w_o):
    """Row by row: y = W_o o, o being one row of concatenated head outputs."""
    return [matvec_t(w_o, ob) for ob in o]
