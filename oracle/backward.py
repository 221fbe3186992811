"""fp64 gradients of exact attention. Test infrastructure only (see the
package docstring for the rule and the page tags).

The pages name the backward pass's memory strategy, recomputation: the
forward keeps only O and a row statistic, and the backward recomputes the
attention weights instead of storing the N x N matrix ([P1] 9.2 item 2,
[P2] 7). They give no formulas. This module writes out the derivative of the
forward definition (``attention_ref``) by the chain rule, with the weights
materialised, so it is the plain definition of the gradients, not a tiled
algorithm:

  S = scale Q K^T (masked entries -inf), P = softmax_rows(S), O = P V
  dV = P^T dO
  dP = dO V^T
  dS_ij = P_ij (dP_ij - sum_l P_il dP_il)          (Jacobian of softmax)
  dQ = scale dS K,   dK = scale dS^T Q

Rows are processed ``chunk`` at a time only to bound memory: dV and dK are
sums over rows, so the chunks add up to the same totals.
"""

from __future__ import annotations

import numpy as np

from .attention import _check, _f64, scores_ref, softmax_rows_ref


def attention_bwd_ref(q, k, v, do, scale, causal=False, window=(-1, -1), chunk=1024):
    """Return (dQ, dK, dV) as float64 arrays [B, H, N, d] for the loss whose
    gradient with respect to O is ``do`` (same shape as q)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"do must have the shape of q: {do.shape} vs {q.shape}")
    B, H, N, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(r0 + chunk, N))
                s = scores_ref(q[b, h], k[b, h], scale, causal, rows, window)
                p, _, _ = softmax_rows_ref(s)
                g = do[b, h, rows]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, rows] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv
