"""Scalar brute-force versions of the oracle for tiny shapes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pure-Python loops with ``math.tanh`` and ``math.exp``: one logit at a time,
the bias cell looked up by integer division of the two positions, the row
softmax by a max / exp / sum over an explicit list.  It follows the same
definition as ``biased_mqa`` ([AG3090] section "Why stock FlashAttention was
not a drop-in replacement", logit equation and list of requirements) but with
none of its array code, so that an indexing or broadcasting slip in one shows
up against the other.  Only for shapes of a few hundred logits.
"""

from __future__ import annotations

import math

from .biased_mqa import as_f64


def project_brute(pair, weight):
    """bias[h][p][r] = sum over c of pair[p][r][c] * weight[c][h], as nested
    lists ([AG3090] section "Profiling pointed at one very large object")."""
    pair = as_f64(pair)
    weight = as_f64(weight)
    P, P2, C = pair.shape
    H = weight.shape[1]
    out = [[[0.0] * P2 for _ in range(P)] for _ in range(H)]
    for h in range(H):
        for p in range(P):
            for r in range(P2):
                acc = 0.0
                for c in range(C):
                    acc += float(pair[p, r, c]) * float(weight[c, h])
                out[h][p][r] = acc
    return out


def attention_brute(q, k, v, bias, *, scale: float, cap: float, block: int = 16):
    """Output [B][S][Hq][Dv] as nested lists.

    ``q`` [B, S, Hq, Dk], ``k`` [B, S, 1, Dk], ``v`` [B, S, 1, Dv],
    ``bias`` [B, Hq, P, P] (one compact bias per batch item).
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    bias = as_f64(bias)
    B, S, Hq, Dk = q.shape
    Dv = v.shape[-1]
    out = [[[[0.0] * Dv for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                row = []
                for j in range(S):
                    dot = 0.0
                    for t in range(Dk):
                        dot += float(q[b, i, h, t]) * float(k[b, j, 0, t])
                    x = scale * dot + float(bias[b, h, i // block, j // block])
                    row.append(cap * math.tanh(x / cap) if cap != 0.0 else x)
                mx = max(row)
                w = [math.exp(x - mx) for x in row]
                tot = sum(w)
                for t in range(Dv):
                    acc = 0.0
                    for j in range(S):
                        acc += w[j] * float(v[b, j, 0, t])
                    out[b][i][h][t] = acc / tot
    return out
