"""Pins of the split-KV oracle (oracle/splitkv.py) against what the
mathematics fixes: a hand-computed two-key example, the identity "merge of
the partials over any partition of the keys = attention over all keys"
(checked against the plain oracle, itself pinned by brute force), and the
algebraic properties of the merge (empty parts, duplicates, order)."""

import math

import numpy as np
import pytest

from oracle import attention_ref
from oracle.splitkv import merge_ref, partial_ref


def rand_qkv(B, H, N, D, seed):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, N, D)) for _ in range(3))


def test_hand_example_two_keys():
    # one query, keys with scores 0 and ln 3 (scale 1, d = 1), values 1 and 5:
    # full softmax weights 1/4, 3/4, so O = 1/4 + 15/4 = 4 and LSE = ln 4.
    q = np.ones((1, 1, 2, 1))
    k = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 5.0]).reshape(1, 1, 2, 1)
    # query row 1 sees both keys; row 0 is there only to give N = 2
    o1, l1 = partial_ref(q, k, v, 1.0, False, [0, 0], [1, 1])
    o2, l2 = partial_ref(q, k, v, 1.0, False, [1, 1], [2, 2])
    assert o1[0, 0, 1, 0] == 1.0 and l1[0, 0, 1] == 0.0
    assert o2[0, 0, 1, 0] == pytest.approx(5.0, abs=1e-15) and l2[0, 0, 1] == pytest.approx(math.log(3.0), abs=1e-15)
    o, lse = merge_ref(np.stack([o1, o2]), np.stack([l1, l2]))
    assert o[0, 0, 1, 0] == pytest.approx(4.0, abs=1e-14)
    assert lse[0, 0, 1] == pytest.approx(math.log(4.0), abs=1e-14)


def random_cuts(rng, N, S):
    """Per-row cut points 0 = c_0 <= c_1 <= ... <= c_S = N (empty parts allowed)."""
    inner = np.sort(rng.integers(0, N + 1, size=(N, S - 1)), axis=1)
    return np.concatenate([np.zeros((N, 1), np.int64), inner, np.full((N, 1), N)], axis=1)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (7, 3)), (True, (20, -1))])
@pytest.mark.parametrize("S", [1, 2, 3, 7])
def test_merge_of_partials_is_full_attention(causal, window, S):
    rng = np.random.default_rng(S * 10 + causal)
    q, k, v = rand_qkv(2, 2, 45, 16, seed=S)
    cuts = random_cuts(rng, 45, S)
    parts = [partial_ref(q, k, v, 0.3, causal, cuts[:, s], cuts[:, s + 1], window) for s in range(S)]
    o, lse = merge_ref(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, lse_ref = attention_ref(q, k, v, 0.3, causal, window=window)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_partial_over_all_keys_is_attention():
    q, k, v = rand_qkv(1, 3, 30, 8, seed=3)
    o, lse = partial_ref(q, k, v, 0.5, True, np.zeros(30, int), np.full(30, 30))
    o_ref, lse_ref = attention_ref(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_partial_with_no_allowed_key_is_neutral():
    q, k, v = rand_qkv(1, 1, 10, 4, seed=4)
    # causal: keys 5..9 are invisible to rows 0..4
    o, lse = partial_ref(q, k, v, 1.0, True, np.full(10, 5), np.full(10, 10))
    assert (o[0, 0, :5] == 0).all() and np.isneginf(lse[0, 0, :5]).all()
    assert np.isfinite(lse[0, 0, 5:]).all()


def test_merge_properties():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 4, 6))
    lse = rng.standard_normal((3, 4))
    base_o, base_l = merge_ref(o, lse)
    # an empty part (LSE = -inf, O = 0) changes nothing
    o2 = np.concatenate([o, np.zeros((1, 4, 6))])
    l2 = np.concatenate([lse, np.full((1, 4), -np.inf)])
    eo, el = merge_ref(o2, l2)
    np.testing.assert_allclose(eo, base_o, atol=1e-15)
    np.testing.assert_allclose(el, base_l, atol=1e-15)
    # order of the parts does not matter
    po, pl = merge_ref(o[::-1], lse[::-1])
    np.testing.assert_allclose(po, base_o, atol=1e-14)
    np.testing.assert_allclose(pl, base_l, atol=1e-14)
    # one part twice: same O, LSE + ln 2
    do, dl = merge_ref(np.stack([o[0], o[0]]), np.stack([lse[0], lse[0]]))
    np.testing.assert_allclose(do, o[0], atol=1e-15)
    np.testing.assert_allclose(dl, lse[0] + math.log(2.0), atol=1e-15)
    # a single part is returned as is
    so, sl = merge_ref(o[:1], lse[:1])
    np.testing.assert_array_equal(so, o[0])
    np.testing.assert_array_equal(sl, lse[0])
    # all parts empty: O = 0, LSE = -inf
    zo, zl = merge_ref(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert (zo == 0).all() and np.isneginf(zl).all()


def test_merge_weights_follow_lse():
    # two parts whose LSE differ by ln 9: weights 1/10 and 9/10
    o = np.array([[[0.0]], [[10.0]]])
    lse = np.array([[1.0], [1.0 + math.log(9.0)]])
    mo, ml = merge_ref(o, lse)
    assert mo[0, 0] == pytest.approx(9.0, abs=1e-13)
    assert ml[0] == pytest.approx(1.0 + math.log(10.0), abs=1e-14)
