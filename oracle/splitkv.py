"""fp64 oracle for split-KV attention: attention over a subset of the keys
(a partial result) and the log-sum-exp merge of partial results. Test
infrastructure only (see the package docstring for the rule).

The pages name the use (long contexts and inference with a KV cache, [P1]
section 11.2) but give no procedure. What is computed here follows from the
plain definition of [P3] section 1.1. Split a row's allowed keys into
disjoint sets K_1 .. K_S, and let l_s = sum over j in K_s of exp(S_ij) and
l = sum_s l_s. Then the softmax over all keys is sum_s (l_s / l) times the
softmax over K_s. In log form, with LSE_s = ln l_s:
    LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
A part with no allowed key has l_s = 0: LSE_s = -inf, and it contributes
nothing (its O_s is defined as 0).
"""

from __future__ import annotations

import numpy as np

from .attention import _check, _f64, scores_ref


def partial_ref(q, k, v, scale, causal, key_lo, key_hi, window=(-1, -1)):
    """Attention of every query row i restricted to the keys j with
    key_lo[i] <= j < key_hi[i] (and allowed by causal / window).

    q, k, v: [B, H, N, d]; key_lo, key_hi: integer arrays of length N (the
    same ranges for every batch and head). Returns (O_s [B, H, N, d],
    LSE_s [B, H, N]) in float64; a row with no allowed key in its range gets
    O_s = 0 and LSE_s = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v)
    B, H, N, D = q.shape
    lo = np.asarray(key_lo, dtype=np.int64)[:, None]
    hi = np.asarray(key_hi, dtype=np.int64)[:, None]
    j = np.arange(N)[None, :]
    in_range = (j >= lo) & (j < hi)
    out = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            s = np.where(in_range, scores_ref(q[b, h], k[b, h], scale, causal, window=window), -np.inf)
            m = s.max(axis=1)
            live = m > -np.inf
            e = np.exp(s[live] - m[live, None])
            l = e.sum(axis=1)
            out[b, h, live] = (e @ v[b, h]) / l[:, None]
            lse[b, h, live] = m[live] + np.log(l)
    return out, lse


def merge_ref(o_parts, lse_parts):
    """Merge S partial results: o_parts [S, ..., d], lse_parts [S, ...].

    LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, evaluated
    with the largest LSE_s subtracted first. Rows where every part is -inf
    get O = 0 and LSE = -inf.
    """
    o = _f64(o_parts)
    ls = _f64(lse_parts)
    if o.shape[:-1] != ls.shape:
        raise ValueError(f"o_parts {o.shape} and lse_parts {ls.shape} disagree")
    m = ls.max(axis=0)
    live = m > -np.inf
    m_safe = np.where(live, m, 0.0)
    w = np.exp(ls - m_safe[None])  # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    o_out = np.where(live[..., None], (w[..., None] * o).sum(axis=0) / np.where(live, total, 1.0)[..., None], 0.0)
    lse_out = np.where(live, m_safe + np.log(np.where(live, total, 1.0)), -np.inf)
    return o_out, lse_out
