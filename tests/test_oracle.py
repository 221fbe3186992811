"""CPU pins for the fp64 oracle (no GPU).

Each test pins the oracle to something other than itself: 40-digit decimal
brute force, closed forms, invariants of softmax attention, a hand-derived
fixture, and a library routine. A mistake in the oracle (a dropped scale, a
wrong sign, a transposed operand, a mask on the wrong side of the diagonal, a
missing rescale in the recurrence) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    attention_bruteforce,
    attention_ref,
    attention_tiled_ref,
    scores_ref,
    softmax_rows_ref,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_examples.json")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- fixtures --

def test_golden_closed_form_examples():
    """Hand-derived examples (tests/golden/closed_form_examples.json)."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        q = np.array(ex["q"])[None, None]
        k = np.array(ex["k"])[None, None]
        v = np.array(ex["v"])[None, None]
        for causal, key in ((False, "noncausal"), (True, "causal")):
            want_o = np.array(ex[key]["o"])
            want_l = np.array(ex[key]["lse"])
            for fn in (attention_ref, attention_tiled_ref, attention_bruteforce):
                o, lse = fn(q, k, v, ex["scale"], causal)
                np.testing.assert_allclose(o[0, 0], want_o, rtol=0, atol=1e-13, err_msg=f"{ex['name']} {key} {fn.__name__}")
                np.testing.assert_allclose(lse[0, 0], want_l, rtol=0, atol=1e-13, err_msg=f"{ex['name']} {key} {fn.__name__}")


# --------------------------------------------------------- T1 brute force --

@pytest.mark.parametrize("N,D", [(1, 1), (2, 3), (5, 4), (8, 8), (7, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_t1_bruteforce(N, D, causal):
    q, k, v = (rnd((2, 1, N, D), s) for s in (1, 2, 3))
    scale = 1.0 / math.sqrt(D)
    o_bf, l_bf = attention_bruteforce(q, k, v, scale, causal)
    for fn in (attention_ref, attention_tiled_ref):
        o, lse = fn(q, k, v, scale, causal)
        np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_bf, rtol=0, atol=1e-13)


def test_t1_bruteforce_nondefault_scale_and_half_inputs():
    """Inputs stored as float16 are upcast exactly; a non-1/sqrt(d) scale."""
    q, k, v = (rnd((1, 2, 6, 5), s).astype(np.float16) for s in (4, 5, 6))
    o_bf, l_bf = attention_bruteforce(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 0.37, True)
    o, lse = attention_ref(q, k, v, 0.37, True)
    np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l_bf, rtol=0, atol=1e-13)


# ----------------------------------------- T2 tiled == untiled (+ control) --

@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 100, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_t2_tiled_equals_untiled(N, causal):
    D = 16
    q, k, v = (rnd((1, 2, N, D), s) for s in (7, 8, 9))
    scale = 1.0 / math.sqrt(D)
    o_ref, l_ref = attention_ref(q, k, v, scale, causal)
    for Br, Bc in [(64, 64), (1, 1), (7, 5), (16, 64), (128, 32), (N, N)]:
        o, lse = attention_tiled_ref(q, k, v, scale, causal, Br=Br, Bc=Bc)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12, err_msg=f"Br={Br} Bc={Bc}")
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12, err_msg=f"Br={Br} Bc={Bc}")


def _blockwise_softmax_sum(q, k, v, scale, block):
    """Negative control: sums independently normalised per-block softmaxes.

    This is the plausible-looking but wrong blocking of "2.3 FlashAttention
    and IO-aware attention", section 2.1 (no running max, no rescale). The
    oracle must not agree with it.
    """
    B, H, N, D = q.shape
    out = np.zeros_like(q)
    for i in range(0, N, block):
        for j in range(0, N, block):
            s = scale * (q[:, :, i:i + block] @ np.swapaxes(k[:, :, j:j + block], -1, -2))
            e = np.exp(s - s.max(axis=-1, keepdims=True))
            out[:, :, i:i + block] += (e / e.sum(axis=-1, keepdims=True)) @ v[:, :, j:j + block]
    return out


def test_t2_negative_control_rejected():
    q, k, v = (rnd((1, 1, 128, 16), s) for s in (10, 11, 12))
    o_ref, _ = attention_ref(q, k, v, 0.25, False)
    wrong = _blockwise_softmax_sum(q, k, v, 0.25, 64)
    assert np.abs(wrong - o_ref).max() > 1e-2


def test_t2_missing_rescale_rejected():
    """A recurrence that forgets the correction factor c disagrees with the oracle."""
    q, k, v = (rnd((1, 1, 128, 16), s) for s in (13, 14, 15))
    o_ref, _ = attention_ref(q, k, v, 0.5, False)
    qi, kk, vv = q[0, 0], k[0, 0], v[0, 0]
    m = np.full(128, -np.inf)
    l = np.zeros(128)
    o = np.zeros((128, 16))
    for ks in range(0, 128, 32):
        s = 0.5 * (qi @ kk[ks:ks + 32].T)
        m_new = np.maximum(m, s.max(axis=1))
        p = np.exp(s - m_new[:, None])
        l = l + p.sum(axis=1)          # c dropped on purpose
        o = o + p @ vv[ks:ks + 32]
        m = m_new
    assert np.abs(o / l[:, None] - o_ref[0, 0]).max() > 1e-3


# ------------------------------------------------ T3 rows of P sum to one --

@pytest.mark.parametrize("causal", [False, True])
def test_t3_rows_sum_to_one(causal):
    N = 300
    q, k = rnd((N, 32), 16), rnd((N, 32), 17)
    p, m, l = softmax_rows_ref(scores_ref(q, k, 0.2, causal))
    assert np.abs(p.sum(axis=1) - 1).max() <= 1e-14 * N
    assert (p >= 0).all()
    if causal:
        assert (p[np.triu_indices(N, 1)] == 0).all()


# ---------------------------------------------------- T4 identical keys --

@pytest.mark.parametrize("causal", [False, True])
def test_t4_identical_keys_give_mean_of_v(causal):
    N, D = 50, 8
    q, v = rnd((1, 1, N, D), 18), rnd((1, 1, N, D), 19)
    kvec = rnd((D,), 20)
    k = np.broadcast_to(kvec, (1, 1, N, D)).copy()
    scale = 0.3
    o, lse = attention_ref(q, k, v, scale, causal)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    want = np.cumsum(v[0, 0], axis=0) / counts[:, None] if causal else np.broadcast_to(v[0, 0].mean(axis=0), (N, D))
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], scale * (q[0, 0] @ kvec) + np.log(counts), rtol=0, atol=1e-13)


# ------------------------------------------------------- T5 single key --

def test_t5_single_key_returns_its_value():
    q, k, v = (rnd((3, 2, 1, 7), s) for s in (21, 22, 23))
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.8, causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse, 0.8 * (q * k).sum(-1), rtol=0, atol=1e-15)


# ----------------------------------------------------------- T6 scale 0 --

@pytest.mark.parametrize("causal", [False, True])
def test_t6_zero_scale_is_uniform(causal):
    N, D = 40, 6
    q, k, v = (rnd((1, 1, N, D), s) for s in (24, 25, 26))
    o, lse = attention_ref(q, k, v, 0.0, causal)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    want = np.cumsum(v[0, 0], axis=0) / counts[:, None] if causal else np.broadcast_to(v[0, 0].mean(axis=0), (N, D))
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=0, atol=1e-13)


# -------------------------------------------------- T7 causal structure --

def test_t7_causal_prefix_only():
    N, D = 33, 8
    q, k, v = (rnd((1, 1, N, D), s) for s in (27, 28, 29))
    o, lse = attention_ref(q, k, v, 0.4, True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    for i in (0, 5, 31):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, i + 1:] = rnd((N - i - 1, D), 30 + i) * 5
        v2[0, 0, i + 1:] = rnd((N - i - 1, D), 60 + i) * 5
        o2, lse2 = attention_ref(q, k2, v2, 0.4, True)
        np.testing.assert_array_equal(o2[0, 0, :i + 1], o[0, 0, :i + 1])
        np.testing.assert_array_equal(lse2[0, 0, :i + 1], lse[0, 0, :i + 1])
    # the non-causal result depends on later keys
    o_nc, _ = attention_ref(q, k, v, 0.4, False)
    assert np.abs(o_nc[0, 0, 0] - v[0, 0, 0]).max() > 1e-3


# ------------------------------------------------------ T8 key shift --

@pytest.mark.parametrize("causal", [False, True])
def test_t8_key_shift_invariance(causal):
    N, D = 70, 12
    q, k, v = (rnd((1, 2, N, D), s) for s in (31, 32, 33))
    u = rnd((D,), 34)
    scale = 0.25
    o, lse = attention_ref(q, k, v, scale, causal)
    o2, lse2 = attention_ref(q, k + u, v, scale, causal)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * (q @ u), rtol=0, atol=1e-12)


# ------------------------------------------------------ T9 affine V --

@pytest.mark.parametrize("causal", [False, True])
def test_t9_affine_values(causal):
    N, D = 45, 6
    q, k, v = (rnd((1, 1, N, D), s) for s in (35, 36, 37))
    A, bvec = rnd((D, D), 38), rnd((D,), 39)
    o, _ = attention_ref(q, k, v, 0.5, causal)
    # O' = O A + 1 b^T for V' = V A + 1 b^T, because every row of P sums to one
    o2, _ = attention_ref(q, k, v @ A + bvec, 0.5, causal)
    np.testing.assert_allclose(o2, o @ A + bvec, rtol=0, atol=1e-12)
    # the oracle's steps with a value width different from d agree too
    o4, _ = _attn_values(q, k, v @ A[:, :4] + bvec[:4], 0.5, causal)
    np.testing.assert_allclose(o4, o @ A[:, :4] + bvec[:4], rtol=0, atol=1e-12)
    oc, _ = _attn_values(q, k, np.full((1, 1, N, 3), 2.5), 0.5, causal)
    np.testing.assert_allclose(oc, 2.5, rtol=0, atol=1e-14)


def _attn_values(q, k, v, scale, causal):
    """Attention with a value width different from d, via the oracle's steps."""
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    lse = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            p, m, l = softmax_rows_ref(scores_ref(q[b, h], k[b, h], scale, causal))
            out[b, h] = p @ v[b, h]
            lse[b, h] = m + np.log(l)
    return out, lse


# ----------------------------------------------------- T10 permutations --

def test_t10_permutation_equivariance():
    N, D = 60, 10
    q, k, v = (rnd((1, 1, N, D), s) for s in (40, 41, 42))
    o, lse = attention_ref(q, k, v, 0.3, False)
    perm = np.random.default_rng(43).permutation(N)
    o_kv, lse_kv = attention_ref(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    np.testing.assert_allclose(o_kv, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_kv, lse, rtol=0, atol=1e-12)
    o_q, lse_q = attention_ref(q[:, :, perm], k, v, 0.3, False)
    np.testing.assert_allclose(o_q, o[:, :, perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_q, lse[:, :, perm], rtol=0, atol=1e-12)


# ------------------------------------------------------ T11 large logits --

def test_t11_large_logits_pick_the_argmax():
    N, D = 20, 8
    q, k, v = (rnd((1, 1, N, D), s) for s in (44, 45, 46))
    scale = 1e3
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, scale, causal)
        s = scale * (q[0, 0] @ k[0, 0].T)
        if causal:
            s[np.triu_indices(N, 1)] = -np.inf
        top2 = np.sort(s, axis=1)[:, -2:]
        assert (top2[:, 1] - top2[:, 0] > 50).sum() >= N - 2  # scores are well separated
        for i in range(N):
            if top2[i, 1] - top2[i, 0] > 50:
                np.testing.assert_allclose(o[0, 0, i], v[0, 0, np.argmax(s[i])], rtol=0, atol=1e-15)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        np.testing.assert_allclose(lse[0, 0], s.max(axis=1), rtol=1e-12, atol=0)


# ------------------------------------------------ T12 library cross-check --

@pytest.mark.parametrize("causal", [False, True])
def test_t12_torch_sdpa_fp64(causal):
    q, k, v = (rnd((2, 3, 97, 32), s) for s in (47, 48, 49))
    scale = 1.0 / math.sqrt(32)
    o, lse = attention_ref(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, want.numpy(), rtol=0, atol=1e-12)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(97, 97, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------- row sampling --

def test_row_subset_matches_full():
    q, k, v = (rnd((1, 2, 130, 16), s) for s in (50, 51, 52))
    rows = np.array([0, 1, 63, 64, 100, 129])
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.25, causal)
        o_s, lse_s = attention_ref(q, k, v, 0.25, causal, rows=rows)
        np.testing.assert_array_equal(o_s, o[:, :, rows])
        np.testing.assert_array_equal(lse_s, lse[:, :, rows])
        o_c, lse_c = attention_ref(q, k, v, 0.25, causal, chunk=7)
        np.testing.assert_allclose(o_c, o, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse_c, lse, rtol=0, atol=1e-15)


# ------------------------------------------------- local-attention window --
# Reading of [P1] 10.1 window_size=(left, right): key j is allowed for query
# i iff i - left <= j <= i + right, a side of -1 unbounded; with causal the
# two masks intersect.

WINDOWS = [(0, 0), (1, 0), (0, 1), (2, 3), (3, -1), (-1, 2), (5, 5)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window_bruteforce(window, causal):
    """The window mask against the decimal brute force, which skips keys
    with its own comparisons."""
    N, D = 8, 4
    q, k, v = (rnd((1, 2, N, D), s) for s in (31, 32, 33))
    o_bf, l_bf = attention_bruteforce(q, k, v, 0.7, causal, window=window)
    for fn in (attention_ref, attention_tiled_ref):
        kw = dict(Br=3, Bc=2) if fn is attention_tiled_ref else {}
        o, lse = fn(q, k, v, 0.7, causal, window=window, **kw)
        np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-13, err_msg=f"{fn.__name__} {window} {causal}")
        np.testing.assert_allclose(lse, l_bf, rtol=0, atol=1e-13, err_msg=f"{fn.__name__} {window} {causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_width_is_identity(causal):
    """window (0, 0): a row sees only its own key, so O_i = V_i exactly and
    LSE_i = scale q_i . k_i (closed form)."""
    N, D = 37, 8
    q, k, v = (rnd((2, 3, N, D), s) for s in (41, 42, 43))
    for fn in (attention_ref, attention_tiled_ref):
        o, lse = fn(q, k, v, 0.3, causal, window=(0, 0))
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, 0.3 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_sequence_is_full_attention(causal):
    """A window at least N wide on both sides masks nothing beyond causal."""
    N, D = 50, 16
    q, k, v = (rnd((1, 2, N, D), s) for s in (51, 52, 53))
    o0, l0 = attention_ref(q, k, v, 0.25, causal)
    for window in ((N, N), (N - 1, N - 1), (-1, N), (N, -1)):
        o, lse = attention_ref(q, k, v, 0.25, causal, window=window)
        np.testing.assert_array_equal(o, o0)
        np.testing.assert_array_equal(lse, l0)


def test_window_weights_vanish_outside_and_sum_to_one():
    """With V = identity (one column per key), O is the weight matrix P: its
    rows sum to 1 and it is exactly 0 outside the band."""
    N = 20
    q, k = rnd((1, 1, N, N), 61) * 0.5, rnd((1, 1, N, N), 62) * 0.5
    v = np.eye(N)[None, None]
    for causal in (False, True):
        for left, right in ((2, 1), (4, -1), (-1, 3), (0, 5)):
            p, _ = attention_ref(q, k, v, 0.9, causal, window=(left, right))
            p = p[0, 0]
            i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
            out = np.zeros_like(p, dtype=bool)
            if left >= 0:
                out |= j < i - left
            if right >= 0:
                out |= j > i + right
            if causal:
                out |= j > i
            assert np.all(p[out] == 0.0), (left, right, causal)
            assert np.all(p[~out] > 0.0), (left, right, causal)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_window_locality():
    """Changing keys and values outside row i's window leaves row i unchanged."""
    N, D, i, left, right = 40, 8, 21, 3, 2
    q, k, v = (rnd((1, 1, N, D), s) for s in (71, 72, 73))
    o0, l0 = attention_ref(q, k, v, 0.5, False, window=(left, right))
    k2, v2 = k.copy(), v.copy()
    far = [j for j in range(N) if j < i - left or j > i + right]
    k2[0, 0, far] = rnd((len(far), D), 74) * 5
    v2[0, 0, far] = rnd((len(far), D), 75) * 5
    o1, l1 = attention_ref(q, k2, v2, 0.5, False, window=(left, right))
    np.testing.assert_array_equal(o1[0, 0, i], o0[0, 0, i])
    np.testing.assert_array_equal(l1[0, 0, i], l0[0, 0, i])
    assert not np.allclose(o1[0, 0, 0], o0[0, 0, 0])  # row 0's window does see the change


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [(5, 0), (0, 7), (13, 9), (64, -1), (-1, 70), (100, 100)])
def test_window_tiled_equals_untiled(window, causal):
    N, D = 150, 8
    q, k, v = (rnd((1, 2, N, D), s) for s in (81, 82, 83))
    o0, l0 = attention_ref(q, k, v, 0.35, causal, window=window)
    for Br, Bc in ((64, 64), (17, 23)):
        o, lse = attention_tiled_ref(q, k, v, 0.35, causal, Br=Br, Bc=Bc, window=window)
        np.testing.assert_allclose(o, o0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l0, rtol=0, atol=1e-12)


def test_window_rejects_sides_below_minus_one():
    q = rnd((1, 1, 4, 2), 91)
    with pytest.raises(ValueError):
        attention_ref(q, q, q, 1.0, False, window=(-2, 0))


# --------------------------------------- fewer queries than keys (Nq < Nk) --

RECT_CASES = [(c, w, nq, nk) for c, w in ((False, (-1, -1)), (True, (-1, -1)), (False, (2, 1)), (True, (3, -1)))
              for nq, nk in ((1, 7), (3, 8), (5, 5), (6, 2))
              if nq <= nk or (not c and w == (-1, -1))]  # Nq > Nk with a mask leaves rows without keys


@pytest.mark.parametrize("causal,window,nq,nk", RECT_CASES)
def test_rectangular_against_bruteforce(causal, window, nq, nk):
    """q [.., Nq, d] against k, v [.., Nk, d]: the queries are the last Nq
    positions. (Rows without keys: test_rectangular_rows_without_keys.)"""
    rng = np.random.default_rng(nq * 10 + nk)
    q = rng.standard_normal((1, 2, nq, 3))
    k = rng.standard_normal((1, 2, nk, 3))
    v = rng.standard_normal((1, 2, nk, 3))
    o, lse = attention_ref(q, k, v, 0.7, causal, window=window)
    ob, lb = attention_bruteforce(q, k, v, 0.7, causal, window=window)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (40, 3)), (True, (17, -1)), (False, (-1, -1))])
def test_rectangular_is_the_last_rows_of_the_square_problem(causal, window):
    """Attention of the last Nq queries against all Nk keys equals rows
    Nk - Nq .. Nk - 1 of the square problem (bottom-right placement)."""
    rng = np.random.default_rng(5)
    nk, nq = 150, 37
    q = rng.standard_normal((2, 2, nk, 16))
    k = rng.standard_normal((2, 2, nk, 16))
    v = rng.standard_normal((2, 2, nk, 16))
    o_sq, l_sq = attention_ref(q, k, v, 0.25, causal, window=window)
    o_r, l_r = attention_ref(q[:, :, nk - nq:], k, v, 0.25, causal, window=window)
    np.testing.assert_allclose(o_r, o_sq[:, :, nk - nq:], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l_r, l_sq[:, :, nk - nq:], rtol=0, atol=1e-15)


def test_rectangular_single_query_sees_every_key_when_causal():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 1, 8))
    k = rng.standard_normal((1, 1, 40, 8))
    v = rng.standard_normal((1, 1, 40, 8))
    a = attention_ref(q, k, v, 0.3, True)
    b = attention_ref(q, k, v, 0.3, False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rectangular_rows_without_keys():
    """Nq > Nk with a causal mask: query i sits at position i - (Nq - Nk),
    so the first Nq - Nk rows see no key: O = 0, LSE = -inf. The others
    equal the square problem on the last Nk queries."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 10, 4))
    k = rng.standard_normal((1, 1, 6, 4))
    v = rng.standard_normal((1, 1, 6, 4))
    o, lse = attention_ref(q, k, v, 0.5, True)
    assert (o[0, 0, :4] == 0).all() and np.isneginf(lse[0, 0, :4]).all()
    o_sq, l_sq = attention_ref(q[:, :, 4:], k, v, 0.5, True)
    np.testing.assert_array_equal(o[:, :, 4:], o_sq)
    np.testing.assert_array_equal(lse[:, :, 4:], l_sq)
