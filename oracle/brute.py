"""Pure-Python brute force for tiny inputs (T <= 16): scalar loops with math.exp.

TEST INFRASTRUCTURE ONLY (see oracle/saf_oracle.py). It exists to cross-check the
vectorised oracle with code that shares nothing with it, not even numpy.

Definitions follow the same page as the vectorised oracle ("When Can Attention Heads Be
Statically Defined?: 中文精读笔记"): part 一 for an ordinary causal softmax head and
part 二.3, Eq. (3) for the compact static pattern, 0-indexed with the diagonal included.
"""
from __future__ import annotations

import math


def _tolist2(x):
    return [[float(c) for c in row] for row in x]


def dynamic_head(q, k, v, scale):
    """One ordinary head: returns (O as list of rows, lse list)."""
    q, k, v = _tolist2(q), _tolist2(k), _tolist2(v)
    T, D = len(q), len(q[0])
    out, lse = [], []
    for i in range(T):
        logits = []
        for j in range(i + 1):
            s = 0.0
            for c in range(D):
                s += q[i][c] * k[j][c]
            logits.append(scale * s)
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        z = sum(w)
        row = [0.0] * len(v[0])
        for j in range(i + 1):
            for c in range(len(v[0])):
                row[c] += w[j] / z * v[j][c]
        out.append(row)
        lse.append(m + math.log(z))
    return out, lse


def frozen_head(alpha, rho, v):
    """One frozen head, Eq. (3): returns (O rows, logZ list, P rows)."""
    alpha = [float(a) for a in alpha]
    rho = [float(r) for r in rho]
    v = _tolist2(v)
    T = len(v)
    out, logz, P = [], [], []
    for i in range(T):
        w = [math.exp(alpha[j] + rho[i - j]) for j in range(i + 1)]
        z = sum(w)
        prow = [w[j] / z if j <= i else 0.0 for j in range(T)]
        row = [0.0] * len(v[0])
        for j in range(i + 1):
            for c in range(len(v[0])):
                row[c] += prow[j] * v[j][c]
        out.append(row)
        logz.append(math.log(z))
        P.append(prow)
    return out, logz, P
