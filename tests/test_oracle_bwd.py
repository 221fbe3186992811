"""CPU pins for the fp64 attention gradients (no GPU).

attention_bwd_ref writes out the chain rule; these tests pin it to things
other than itself: central finite differences of the forward oracle (the
definition of a derivative), torch autograd through a plain float64 torch
attention, closed forms, and invariants of softmax attention. A dropped
softmax-Jacobian term, a transposed weight matrix, a missing scale or a mask
on the wrong side fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_ref, allowed_ref


def rnd(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def loss(q, k, v, g, scale, causal, window):
    o, _ = attention_ref(q, k, v, scale, causal, window=window)
    return float((o * g).sum())


CASES = [(False, (-1, -1)), (True, (-1, -1)), (False, (2, 1)), (True, (3, -1))]


@pytest.mark.parametrize("causal,window", CASES)
def test_directional_finite_differences(causal, window):
    """<grad, E> against (L(x + eps E) - L(x - eps E)) / (2 eps) for random
    directions E, for each of q, k, v (loss L = sum O * G)."""
    B, H, N, D = 1, 2, 9, 5
    q, k, v, g = (rnd((B, H, N, D), s) for s in (1, 2, 3, 4))
    scale, eps = 0.6, 1e-5
    dq, dk, dv = attention_bwd_ref(q, k, v, g, scale, causal, window)
    for idx, grad in enumerate((dq, dk, dv)):
        for t in range(3):
            e = rnd((B, H, N, D), 100 + 10 * idx + t)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx] = args_p[idx] + eps * e
            args_m[idx] = args_m[idx] - eps * e
            fd = (loss(*args_p, g, scale, causal, window) - loss(*args_m, g, scale, causal, window)) / (2 * eps)
            an = float((grad * e).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (idx, t, fd, an)


def test_elementwise_finite_differences_tiny():
    """Every element of every gradient on a tiny causal case."""
    B, H, N, D = 1, 1, 4, 3
    q, k, v, g = (rnd((B, H, N, D), s) for s in (5, 6, 7, 8))
    scale, eps = 0.9, 1e-6
    grads = attention_bwd_ref(q, k, v, g, scale, True)
    for idx in range(3):
        for pos in np.ndindex(B, H, N, D):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[idx][pos] += eps
            args_m[idx][pos] -= eps
            fd = (loss(*args_p, g, scale, True, (-1, -1)) - loss(*args_m, g, scale, True, (-1, -1))) / (2 * eps)
            assert abs(fd - grads[idx][pos]) <= 1e-8, (idx, pos, fd, grads[idx][pos])


@pytest.mark.parametrize("causal,window", CASES + [(False, (0, 0))])
def test_torch_autograd_fp64(causal, window):
    """torch autograd through softmax(scale Q K^T + mask) V in float64."""
    B, H, N, D = 2, 2, 33, 16
    q, k, v, g = (rnd((B, H, N, D), s) for s in (11, 12, 13, 14))
    scale = 1 / math.sqrt(D)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    mask = torch.tensor(allowed_ref(np.arange(N), np.arange(N), causal, window))
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(g))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, scale, causal, window)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_zero_width_window_closed_form():
    """window (0, 0): O = V, so dV = dO and dQ = dK = 0 exactly."""
    q, k, v, g = (rnd((1, 3, 20, 8), s) for s in (21, 22, 23, 24))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, 0.4, False, (0, 0))
    np.testing.assert_array_equal(dv, g)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0


def test_single_key_closed_form():
    """N = 1: O = V whatever Q and K are, so dV = dO and dQ = dK = 0."""
    q, k, v, g = (rnd((2, 2, 1, 16), s) for s in (31, 32, 33, 34))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, 1.3, True)
    np.testing.assert_array_equal(dv, g)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0


@pytest.mark.parametrize("causal,window", CASES)
def test_key_gradients_sum_to_zero(causal, window):
    """Each row of dS sums to 0 (softmax is shift invariant), so
    sum_j dK_j = scale sum_i (sum_j dS_ij) q_i = 0."""
    q, k, v, g = (rnd((1, 2, 40, 8), s) for s in (41, 42, 43, 44))
    _, dk, _ = attention_bwd_ref(q, k, v, g, 0.7, causal, window)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12


def test_shifting_all_keys_leaves_dq_unchanged():
    """Adding one vector c to every key adds scale q.c to a whole row of S,
    which softmax ignores, and dQ = scale dS K changes by scale (sum_j dS_ij) c = 0."""
    q, k, v, g = (rnd((1, 1, 25, 8), s) for s in (51, 52, 53, 54))
    c = rnd((8,), 55, 3.0)
    dq0, _, dv0 = attention_bwd_ref(q, k, v, g, 0.5, True)
    dq1, _, dv1 = attention_bwd_ref(q, k + c, v, g, 0.5, True)
    np.testing.assert_allclose(dq1, dq0, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv1, dv0, rtol=0, atol=1e-11)


def test_dv_is_linear_in_do_and_independent_of_v():
    q, k, v, g1, g2 = (rnd((1, 2, 30, 8), s) for s in (61, 62, 63, 64, 65))
    _, _, dv1 = attention_bwd_ref(q, k, v, g1, 0.5, False)
    _, _, dv2 = attention_bwd_ref(q, k, v * 3 + 1, g2, 0.5, False)
    _, _, dv12 = attention_bwd_ref(q, k, v, 2 * g1 - g2, 0.5, False)
    np.testing.assert_allclose(dv12, 2 * dv1 - dv2, rtol=0, atol=1e-12)


def test_row_chunking_does_not_change_the_result():
    q, k, v, g = (rnd((1, 2, 70, 8), s) for s in (71, 72, 73, 74))
    a = attention_bwd_ref(q, k, v, g, 0.5, True, chunk=1024)
    b = attention_bwd_ref(q, k, v, g, 0.5, True, chunk=16)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


def test_planted_jacobian_mistake_is_caught():
    """Negative control: dropping the row term of the softmax Jacobian
    (dS = P dP) gives gradients the finite differences reject."""
    B, H, N, D = 1, 1, 6, 4
    q, k, v, g = (rnd((B, H, N, D), s) for s in (81, 82, 83, 84))
    from oracle.attention import scores_ref, softmax_rows_ref

    p, _, _ = softmax_rows_ref(scores_ref(q[0, 0], k[0, 0], 0.8, False))
    wrong_dq = 0.8 * ((p * (g[0, 0] @ v[0, 0].T)) @ k[0, 0])
    e = rnd((B, H, N, D), 85)
    eps = 1e-5
    fd = (loss(q + eps * e, k, v, g, 0.8, False, (-1, -1)) - loss(q - eps * e, k, v, g, 0.8, False, (-1, -1))) / (2 * eps)
    assert abs(fd - float((wrong_dq * e[0, 0]).sum())) > 1e-3
