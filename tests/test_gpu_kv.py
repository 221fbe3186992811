"""GPU parity for fewer queries than keys (fa_fwd_kv): N query rows against
an Nk-row key/value cache, the queries being the last N positions. The
oracle (attention_ref with k, v of Nk rows, pinned in test_oracle.py)
decides; bounds as in test_gpu_parity.py. Outputs are pre-filled with NaN."""

import math
import sys

import numpy as np
import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs
from oracle import attention_ref

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1e-2, torch.float32: 1e-5}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not fabuild.is_built():
        fabuild.build()
    fa.lib()


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def make(B, H, N, Nk, D, dtype, seed):
    q = inputs.make_qkv(B, H, N, D, dtype, seed=seed)[0]
    _, k, v = inputs.make_qkv(B, H, Nk, D, dtype, seed=seed + 1)
    return q, k, v


def run(q, k, v, causal, window=(-1, -1), splits=1):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(qd, kd, vd, causal=causal, window_size=window, out=o, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, q, k, v, causal, window=(-1, -1)):
    scale = 1.0 / math.sqrt(q.shape[-1])
    o_ref, l_ref = attention_ref(np64(q), np64(k), np64(v), scale, causal, window=window)
    assert np.isfinite(np64(o)).all() and np.isfinite(np64(lse)).all()
    err_o = np.abs(np64(o) - o_ref).max()
    err_l = np.abs(np64(lse) - l_ref).max()
    assert err_o <= TOL_O[q.dtype], err_o
    assert err_l <= TOL_LSE, err_l


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("N,Nk", [(1, 1000), (7, 300), (130, 777), (300, 301)])
def test_fewer_queries(dtype, D, N, Nk):
    for causal in (False, True):
        q, k, v = make(1, 2, N, Nk, D, dtype, seed=N + Nk + D)
        o, lse = run(q, k, v, causal)
        check(o, lse, q, k, v, causal)


@pytest.mark.parametrize("window", [(64, 0), (10, 5), (300, -1)])
def test_fewer_queries_window(window):
    q, k, v = make(2, 2, 90, 700, 128, "bf16", seed=3)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, window)
        check(o, lse, q, k, v, causal, window)


def test_more_queries_than_keys_without_mask():
    q, k, v = make(1, 3, 500, 200, 64, "f16", seed=5)
    o, lse = run(q, k, v, False)
    check(o, lse, q, k, v, False)


@pytest.mark.parametrize("splits", [0, 3, 16])
def test_decode_step_with_split_kv(splits):
    """One new token per head against a 32k cache (B=1, H=8, d=128, bf16,
    causal): the key range is split across workgroups."""
    q, k, v = make(1, 8, 1, 32768, 128, "bf16", seed=9)
    o, lse = run(q, k, v, True, splits=splits)
    check(o, lse, q, k, v, True)


def test_cache_layout_in_place():
    """q [B, 4, H, d] and a [B, Nk, H, d] cache as strided views."""
    B, N, Nk, H, D = 2, 4, 1500, 6, 128
    qb = inputs.make_qkv(B, N, H, D, "bf16", seed=11)[0].cuda()       # [B, N, H, D]
    kb, vb = (t.cuda() for t in inputs.make_qkv(B, Nk, H, D, "bf16", seed=12)[1:])  # [B, Nk, H, D]
    o = fa.flash_attn_func(qb, kb, vb, causal=True)
    assert o.shape == (B, N, H, D)
    torch.cuda.synchronize()
    qc, kc, vc = (t.transpose(1, 2).contiguous().cpu() for t in (qb, kb, vb))
    _, lse = fa.fwd(*(t.transpose(1, 2) for t in (qb, kb, vb)), causal=True)
    check(o.transpose(1, 2).cpu(), lse.cpu(), qc, kc, vc, True)


def test_rectangular_equals_last_rows_of_square():
    """The rectangular call agrees with the last N rows of the square call
    on the same keys (within the forward's bound; the two calls group rows
    into different query tiles)."""
    Nk, N = 1000, 200
    q, k, v = inputs.make_qkv(1, 2, Nk, 128, "bf16", seed=13)
    o_sq, l_sq = run(q, k, v, True)
    o_r, l_r = run(q[:, :, Nk - N:].contiguous(), k, v, True)
    assert (o_r.float() - o_sq[:, :, Nk - N:].float()).abs().max().item() <= TOL_O[torch.bfloat16]
    assert (l_r - l_sq[:, :, Nk - N:]).abs().max().item() <= 1e-5


def test_backward_needs_equal_lengths():
    q, k, v = (t.cuda().requires_grad_(True) for t in make(1, 1, 8, 16, 64, "bf16", seed=1))
    o = fa.attention(q, k, v)
    with pytest.raises(NotImplementedError):
        o.sum().backward()
