"""CPU checks of the rounding model (tests/kernel_model.py) against the fp64
oracle, so that the GPU comparison with the model rests on a model that is
itself right:

* without its two 16-bit roundings (exact=True, float64) the model's tiled
  recurrence with the lazy exponent reference must reproduce the plain
  definition to float64 rounding, on shapes that exercise every branch
  (ragged tiles, causal, windows, fewer queries than keys, zero and negative
  scales, keys whose norms grow so that rows move their reference);
* with them, its error against the oracle must stay within the worst case of
  those two roundings, u (A + |O|) per element (A = softmax over |V|), and
  reach a sizeable share of it (the roundings are really there);
* a row that sees one key returns that key's value exactly.
"""

import math

import numpy as np
import pytest
import torch

from kernel_model import forward_model, output_ulp
from oracle import attention_ref
from transformer_exact_attention_flashattention_amd import inputs

U16 = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}

CASES = [
    # B, H, N, Nk, D, dtype, causal, window, scale multiplier
    (1, 2, 300, 300, 64, "bf16", True, (-1, -1), 1.0),
    (2, 1, 257, 257, 128, "f16", False, (-1, -1), 1.0),
    (1, 1, 700, 700, 64, "bf16", True, (300, -1), 1.0),
    (1, 2, 257, 700, 64, "f16", False, (80, 7), 1.0),
    (1, 1, 130, 777, 128, "bf16", True, (-1, -1), 1.0),
    (1, 1, 200, 200, 64, "bf16", True, (5, -1), -1.0),
    (1, 1, 130, 130, 64, "f16", False, (-1, -1), 0.0),
    (1, 1, 65, 65, 256, "bf16", False, (0, 3), 2.5),
]


def _draw(B, H, N, Nk, D, dtype, seed):
    q = inputs.make_qkv(B, H, N, D, dtype, seed=seed)[0]
    _, k, v = inputs.make_qkv(B, H, Nk, D, dtype, seed=seed + 1)
    return q, k, v


def _np(t):
    return t.double().numpy()


@pytest.mark.parametrize("case", CASES)
def test_exact_model_is_the_definition(case):
    B, H, N, Nk, D, dtype, causal, window, smul = case
    q, k, v = _draw(B, H, N, Nk, D, dtype, seed=N + D)
    scale = smul / math.sqrt(D)
    o, lse = forward_model(q, k, v, scale, causal, window, exact=True)
    o_ref, l_ref = attention_ref(_np(q), _np(k), _np(v), scale, causal, window=window)
    assert np.abs(o.numpy() - o_ref).max() <= 1e-12
    assert np.abs(lse.numpy() - l_ref).max() <= 1e-12


@pytest.mark.parametrize("exact", [True, False])
def test_growing_logits_move_the_reference(exact):
    """Key norms growing x0.05 .. x4 at twice the default scale: later tiles'
    scores exceed the first tile's maximum by far more than 2^8 allows, so
    rows move their reference; the exact model still equals the definition
    and the rounded one stays within its rounding bound."""
    N, D = 700, 128
    q, k, v = inputs.make_qkv(1, 2, N, D, "bf16", seed=21)
    k = (k.float() * torch.linspace(0.05, 4.0, N).view(1, 1, N, 1)).to(k.dtype)
    scale = 2.0 / math.sqrt(D)
    o, _ = forward_model(q, k, v, scale, True, exact=exact)
    o_ref, _ = attention_ref(_np(q), _np(k), _np(v), scale, True)
    if exact:
        assert np.abs(o.numpy() - o_ref).max() <= 1e-12
    else:
        a, _ = attention_ref(_np(q), _np(k), np.abs(_np(v)), scale, True)
        assert (np.abs(_np(o) - o_ref) <= U16[q.dtype] * (a + np.abs(o_ref)) + 1e-6).all()


@pytest.mark.parametrize("case", CASES)
def test_rounded_model_within_its_rounding_bound(case):
    B, H, N, Nk, D, dtype, causal, window, smul = case
    q, k, v = _draw(B, H, N, Nk, D, dtype, seed=N + D)
    scale = smul / math.sqrt(D)
    o, lse = forward_model(q, k, v, scale, causal, window)
    assert o.dtype == q.dtype
    o_ref, l_ref = attention_ref(_np(q), _np(k), _np(v), scale, causal, window=window)
    a, _ = attention_ref(_np(q), _np(k), np.abs(_np(v)), scale, causal, window=window)
    bound = U16[q.dtype] * (a + np.abs(o_ref)) + 1e-6
    err = np.abs(_np(o) - o_ref)
    assert (err <= bound).all()
    assert (err / bound).max() > 0.1  # the 16-bit roundings are really applied
    assert np.abs(lse.double().numpy() - l_ref).max() <= 1e-5


def test_one_visible_key_returns_its_value():
    q, k, v = inputs.make_qkv(2, 2, 300, 64, "bf16", seed=3)
    o, _ = forward_model(q, k, v, 0.125, False, (0, 0))
    assert torch.equal(o, v)
    o, _ = forward_model(q, k, v, 0.125, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])


def test_output_ulp():
    o = np.array([1.0, 1.5, 2.0, 0.75, -3.0, 0.0])
    assert np.array_equal(output_ulp(o, torch.bfloat16), [2 ** -7, 2 ** -7, 2 ** -6, 2 ** -8, 2 ** -6, 2.0 ** -133])
    assert np.array_equal(output_ulp(o, torch.float16)[:3], [2 ** -10, 2 ** -10, 2 ** -9])
