"""Brute-force attention in 40-digit decimal arithmetic, for tiny inputs.

Test infrastructure only (see the package docstring). It writes the softmax
straight from its definition, exp(S_ij) / sum_j exp(S_ij), with no max
subtraction and no float64 arithmetic, so that it pins the fp64 oracle with
an independent route: [P3] 1.1 (scores, -inf mask, softmax, times V) and
[P5] ``standard_attention``. Pure-Python loops: keep N and d small (N <= 8).
"""

from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np


def attention_bruteforce(q, k, v, scale, causal=False, digits=40, window=(-1, -1)):
    """Return (O, LSE) as float64 arrays, computed in Decimal at ``digits``.

    Every float input converts to Decimal exactly. k and v may hold more rows
    (Nk) than q (Nq): query i then sits at position p = i + Nk - Nq, the last
    Nq positions of the sequence. A masked key (causal and j > p, or outside
    the window: j < p - left for left >= 0, j > p + right for right >= 0) is
    left out of both sums, which is what a -inf score means.
    """
    left, right = int(window[0]), int(window[1])
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    NK = k.shape[2]
    if N > 64 or NK > 64:
        raise ValueError("brute force is for tiny inputs only")
    out = np.empty((B, H, N, D))
    lse = np.empty((B, H, N))
    with localcontext() as ctx:
        ctx.prec = digits
        sc = Decimal(float(scale))
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    pos = i + NK - N
                    weights = []
                    for j in range(NK):
                        if causal and j > pos:
                            continue
                        if left >= 0 and pos - j > left:
                            continue
                        if right >= 0 and j - pos > right:
                            continue
                        dot = sum((Decimal(float(q[b, h, i, c])) * Decimal(float(k[b, h, j, c]))
                                   for c in range(D)), Decimal(0))
                        weights.append((j, (sc * dot).exp()))
                    total = sum((w for _, w in weights), Decimal(0))
                    for c in range(D):
                        num = sum((w * Decimal(float(v[b, h, j, c])) for j, w in weights), Decimal(0))
                        out[b, h, i, c] = float(num / total)
                    lse[b, h, i] = float(total.ln())
    return out, lse
