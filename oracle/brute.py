"""Pure-Python loop versions of the oracle steps, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  These use nothing but Python floats, ``math.exp``
and ``math.fsum`` (a correctly rounded sum), with explicit loops over every
index, so that a vectorisation mistake in ``oracle.method`` (a wrong axis, a
transposed operand, an off-by-one block) shows up as a disagreement.  They
follow the same readings of the pages as ``oracle.method``.
"""
from __future__ import annotations

import math


def softmax(z):
    mx = max(z)
    e = [math.exp(v - mx) for v in z]
    s = math.fsum(e)
    return [v / s for v in e]


def compress(rows, z, m):
    """rows: list of n lists of d floats (positions 0..n-1)."""
    alpha = softmax(z)
    n = len(rows)
    d = len(rows[0]) if n else 0
    out = []
    for j in range(n // m):
        out.append([math.fsum(alpha[s] * rows[j * m + s][c] for s in range(m)) for c in range(d)])
    return out


def score(q_heads, w_heads, key):
    """sum_h w_h * max(0, q_h . key)."""
    terms = []
    for qh, wh in zip(q_heads, w_heads):
        dot = math.fsum(a * b for a, b in zip(qh, key))
        terms.append(wh * max(0.0, dot))
    return math.fsum(terms)


def topk(scores, k):
    """scores: list of (index, score) over visible entries; ties to the lower index."""
    ordered = sorted(scores, key=lambda p: (-p[1], p[0]))
    return [j for j, _ in ordered[:k]]


def attend(q_heads, keys, values, scale):
    """Per head softmax over the entry list; returns (o [H][d], lse [H])."""
    outs, lses = [], []
    for qh in q_heads:
        if not keys:
            outs.append([0.0] * len(qh))
            lses.append(-math.inf)
            continue
        logits = [scale * math.fsum(a * b for a, b in zip(qh, k)) for k in keys]
        mx = max(logits)
        p = [math.exp(v - mx) for v in logits]
        den = math.fsum(p)
        outs.append([math.fsum(p[e] * values[e][c] for e in range(len(values))) / den
                     for c in range(len(values[0]))])
        lses.append(mx + math.log(den))
    return outs, lses


def csa_query(t, q_heads, kc, vc, selected, k_raw, v_raw, W, m, scale):
    """One CSA query at position t (raw rows start at position 0)."""
    c = min((t + 1) // m, len(kc))
    keys, vals = [], []
    for j in selected:
        if 0 <= j < c:
            keys.append(kc[j])
            vals.append(vc[j])
    for p in range(max(0, t - W + 1), t + 1):
        keys.append(k_raw[p])
        vals.append(v_raw[p])
    return attend(q_heads, keys, vals, scale)


def hca_query(t, q_heads, kc, vc, m_heavy, k_raw, v_raw, W, scale):
    c = min((t + 1) // m_heavy, len(kc))
    keys = [kc[j] for j in range(c)] + [k_raw[p] for p in range(max(0, t - W + 1), t + 1)]
    vals = [vc[j] for j in range(c)] + [v_raw[p] for p in range(max(0, t - W + 1), t + 1)]
    return attend(q_heads, keys, vals, scale)
