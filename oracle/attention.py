"""fp64 oracle: the plain definition of attention and the tiled online-softmax
variant. Test infrastructure only (see the package docstring for the rule and
the page tags [P1]-[P5]).

Inputs are numpy arrays laid out [B, H, N, d] (the layout of [P3] section 1.1),
of any float dtype; they are upcast exactly to float64 before any arithmetic,
so the oracle sees exactly the values that were stored in the input dtype.

Readings of the pages used here (where they are silent or disagree):

* scale is an explicit argument; callers pass 1/sqrt(d) for the default
  ([P1] 5.2 ``softmax_scale=None``; [P5] ``standard_attention`` divides by
  sqrt(d); [P3] 1.1 has no scale at all, which is the case scale = 1).
* causal means key j is allowed for query i iff j <= i: the lower-triangular
  mask, written as a -inf fill before the softmax ([P3] 1.1). Query and key
  lengths are equal, so every row keeps at least its diagonal key.
* LSE_i = ln sum_j exp(S_ij) over allowed j, in natural log (the pages never
  write it; it is the row statistic m + ln l of the online recurrence).
* window = (left, right) is the local-attention window that [P1] 10.1 lists
  as ``window_size=(-1, -1)`` without defining it: key j is allowed for query
  i iff j >= i - left (when left >= 0) and j <= i + right (when right >= 0);
  -1 leaves that side unbounded, so (-1, -1) is full attention. It combines
  with causal by intersection. The diagonal key is always allowed, so no row
  is empty.
* Fewer queries than keys (Nq < Nk: new tokens against a key/value cache,
  the inference use of [P1] 11.2, which the pages do not define): the Nq
  queries are the last Nq positions of the Nk-long sequence, so query row i
  sits at position i + Nk - Nq and the causal and window tests above apply
  to that position. With Nq = Nk this is the definition above. A row with no
  allowed key (possible only with Nq > Nk) gets O = 0 and LSE = -inf.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype.kind != "f":
        raise TypeError(f"oracle expects a float array, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def _check(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B,H,N,d] shape: {q.shape} {k.shape} {v.shape}")


def _check_kv(q, k, v):
    """q [B, H, Nq, d]; k, v [B, H, Nk, d] (Nk may differ from Nq)."""
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"q must be [B,H,Nq,d] and k, v [B,H,Nk,d]: {q.shape} {k.shape} {v.shape}")


def _check_window(window):
    left, right = (int(w) for w in window)
    if left < -1 or right < -1:
        raise ValueError(f"window sides must be >= -1 (-1: unbounded), got {window}")
    return left, right


def allowed_ref(rows, keys, causal, window=(-1, -1), offset=0):
    """Boolean [len(rows), len(keys)]: may query row i attend to key j?

    Query row i sits at position i + offset (offset = Nk - Nq, the reading
    for fewer queries than keys in the module docstring; 0 when the lengths
    are equal). causal: j <= i ([P3] 1.1 lower-triangular mask). window
    (left, right): j >= i - left and j <= i + right, each side only when
    >= 0 (the reading of [P1] 10.1 ``window_size``), with i the position.
    """
    left, right = _check_window(window)
    i = np.asarray(rows, dtype=np.int64)[:, None] + int(offset)
    j = np.asarray(keys, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        ok &= j <= i
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


def scores_ref(q_bh, k_bh, scale, causal, rows=None, window=(-1, -1)):
    """S = scale * Q K^T for one (batch, head), masked entries set to -inf.

    Step 1 of standard attention ([P3] 1.1, [P2] 2, [P5] standard_attention):
    S_ij = scale * sum_c Q_ic K_jc. Entries a row may not attend to (causal:
    j > i; outside the window) are filled with -inf ([P3] 1.1
    ``masked_fill``). ``rows`` selects query rows (default: all); the
    returned S has one row per selected query and one column per key.
    """
    q_bh = _f64(q_bh)
    k_bh = _f64(k_bh)
    n = k_bh.shape[0]
    rows = np.arange(q_bh.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    s = float(scale) * (q_bh[rows] @ k_bh.T)
    if causal or tuple(window) != (-1, -1):
        s = np.where(allowed_ref(rows, np.arange(n), causal, window, n - q_bh.shape[0]), s, -np.inf)
    return s


def softmax_rows_ref(s):
    """Row softmax of S with the row max subtracted first (step 2 of [P3] 1.1).

    Returns (P, m, l): m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i),
    P_ij = exp(S_ij - m_i) / l_i. Masked (-inf) entries give exactly 0.
    """
    m = s.max(axis=1, keepdims=True)
    empty = np.isneginf(m[:, 0])
    e = np.exp(s - np.where(empty[:, None], 0.0, m))
    l = e.sum(axis=1, keepdims=True)
    p = np.where(empty[:, None], 0.0, e / np.where(empty[:, None], 1.0, l))
    return p, m[:, 0], l[:, 0]


def attention_ref(q, k, v, scale, causal=False, rows=None, chunk=1024, window=(-1, -1)):
    """Plain three-step attention: O = softmax(scale Q K^T [+ mask]) V, and LSE.

    [P3] 1.1 (QK^T, mask + softmax, times V), [P2] 2 and [P5]
    ``standard_attention``. q is [B, H, Nq, d] and k, v are [B, H, Nk, d]
    (Nk = Nq unless a key/value cache is longer; see the module docstring
    for where the queries then sit). Returns (O, LSE) as float64 arrays of
    shape [B, H, R, d] and [B, H, R], where R is the number of selected query
    rows (all Nq by default). Query rows are processed ``chunk`` at a time
    only to bound memory; each chunk is the same untiled computation over all
    keys. LSE_i = m_i + ln l_i = ln sum_j exp(S_ij).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_kv(q, k, v)
    B, H, N, D = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.empty((B, H, R, D), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for c0 in range(0, R, chunk):
                rr = rows[c0:c0 + chunk]
                s = scores_ref(q[b, h], k[b, h], scale, causal, rr, window)
                p, m, l = softmax_rows_ref(s)
                out[b, h, c0:c0 + chunk] = p @ v[b, h]
                lse[b, h, c0:c0 + chunk] = np.where(np.isneginf(m), -np.inf, m + np.log(np.where(l > 0, l, 1.0)))
    return out, lse


def attention_tiled_ref(q, k, v, scale, causal=False, Br=64, Bc=64, window=(-1, -1)):
    """Tiled forward with the online-softmax recurrence, in float64.

    Follows [P5] ``flash_attention_forward``: for each block of Br query rows,
    start from m = -inf, l = 0, O = 0; for each block of Bc keys/values:
    S = scale * Q_i K_j^T (masked entries -inf, as in [P3] 1.1);
    (1) m_new = max(m, rowmax S); (2) P = exp(S - m_new);
    (3) c = exp(m - m_new); (4) l = c l + rowsum P, O = c O + P V_j;
    (5) m = m_new. After the last block, O / l. Ragged last blocks are cut
    at N, as the page's ``min(start + block, N)`` does.

    One addition the page does not need (it has no mask): while every key a
    row has seen so far is masked, m_new stays -inf and exp(-inf - (-inf))
    would be NaN, so such rows keep their state (c = 1, P = 0) for that
    block. The LSE of a row is m + ln l after the last block. ``window`` as
    in ``attention_ref``; with it a row's first blocks can be fully masked,
    which the same guard covers.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v)
    B, H, N, D = q.shape
    out = np.zeros((B, H, N, D), dtype=np.float64)
    lse = np.zeros((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for qs in range(0, N, Br):
                qe = min(qs + Br, N)
                qi = q[b, h, qs:qe]
                m = np.full(qe - qs, -np.inf)
                l = np.zeros(qe - qs)
                o = np.zeros((qe - qs, D))
                for ks in range(0, N, Bc):
                    ke = min(ks + Bc, N)
                    s = float(scale) * (qi @ k[b, h, ks:ke].T)
                    if causal or tuple(window) != (-1, -1):
                        allowed = allowed_ref(np.arange(qs, qe), np.arange(ks, ke), causal, window)
                        s = np.where(allowed, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)
                    base = np.where(live, m_new, 0.0)
                    p = np.where(live[:, None], np.exp(s - base[:, None]), 0.0)
                    c = np.where(live, np.exp(m - base), 1.0)
                    l = c * l + p.sum(axis=1)
                    o = c[:, None] * o + p @ v[b, h, ks:ke]
                    m = m_new
                out[b, h, qs:qe] = o / l[:, None]
                lse[b, h, qs:qe] = m + np.log(l)
    return out, lse
