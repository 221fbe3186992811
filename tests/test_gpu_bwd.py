"""GPU parity of the backward pass (fa_bwd) against the fp64 gradient oracle.

Bar: max |dX - dX_oracle| <= tol * max(max |dX_oracle|, 1) for dX in dQ, dK,
dV, with tol = 1e-2 for bf16 and 2e-3 for fp16 inputs: the forward's bounds,
applied relative to each gradient's largest magnitude because gradients are
not normalised the way O is (|O| <= max |V|). The inputs have unit variance,
so gradients are of order 1; the floor of 1 keeps a gradient that vanishes
exactly (one key, a zero-width window), where the kernel's two fp32 routes to
dP and delta differ by rounding only, from turning that noise into an
infinite relative error. Every gradient element passes
through two roundings to the input type (a matrix-core operand, P or dS, and
the output itself) after fp32 accumulation, about 2 units of bf16 (7.8e-3) or
fp16 (9.8e-4) rounding. The forward outputs o and lse fed to the backward
come from the HIP forward; the oracle recomputes everything from q, k, v and
do in fp64.
"""

import math
import sys

import numpy as np
import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f16": 2e-3}


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


def make(B, H, N, D, dtype, seed):
    q, k, v = inputs.make_qkv(B, H, N, D, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    return q, k, v, do


def run_bwd(q, k, v, do, scale, causal, window=(-1, -1)):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, softmax_scale=scale, causal=causal, window_size=window)
    outs = [torch.full_like(qd, float("nan")) for _ in range(3)]
    delta = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, softmax_scale=scale, causal=causal, window_size=window,
                        dq=outs[0], dk=outs[1], dv=outs[2], delta=delta)
    torch.cuda.synchronize()
    return [t.cpu() for t in (dq, dk, dv)], o.cpu(), delta.cpu()


def check(grads, q, k, v, do, scale, causal, window, dtype):
    ref = attention_bwd_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                            scale, causal, window)
    for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
        g = got.double().numpy()
        assert np.isfinite(g).all(), f"{name}: unwritten or non-finite"
        err = np.abs(g - r).max() / max(np.abs(r).max(), 1.0)
        assert err <= TOL[dtype], f"{name}: max|d| / max(max|ref|, 1) = {err:.3e} > {TOL[dtype]:.0e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_lengths(dtype, D, causal):
    """Single and partial tiles, exact multiples of the 64-row and 128-row
    tiles, and ragged tails."""
    for N in (1, 2, 31, 64, 100, 128, 129, 257, 500):
        q, k, v, do = make(1, 2, N, D, dtype, seed=N + D)
        scale = 1.0 / math.sqrt(D)
        grads, _, _ = run_bwd(q, k, v, do, scale, causal)
        check(grads, q, k, v, do, scale, causal, (-1, -1), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_windows(dtype, D):
    for causal, window, N in ((False, (0, 0), 200), (False, (5, 3), 300), (True, (64, 0), 300),
                              (False, (130, -1), 400), (False, (-1, 70), 400), (True, (1000, 1000), 150)):
        q, k, v, do = make(1, 2, N, D, dtype, seed=N + D + window[0])
        scale = 1.0 / math.sqrt(D)
        grads, _, _ = run_bwd(q, k, v, do, scale, causal, window)
        check(grads, q, k, v, do, scale, causal, window, dtype)


@pytest.mark.parametrize("scale", [0.0, -0.4, 1.0])
def test_bwd_other_scales(scale):
    q, k, v, do = make(2, 2, 150, 64, "bf16", seed=3)
    grads, _, _ = run_bwd(q, k, v, do, scale, True)
    check(grads, q, k, v, do, scale, True, (-1, -1), "bf16")


def test_bwd_batch_heads_long_causal():
    """A GPT-3-shaped slice (4 of the 128 heads at N = 2048, d = 128, bf16,
    causal): many key blocks and query tiles per head."""
    q, k, v, do = make(1, 4, 2048, 128, "bf16", seed=42)
    scale = 1.0 / math.sqrt(128)
    grads, _, _ = run_bwd(q, k, v, do, scale, True)
    check(grads, q, k, v, do, scale, True, (-1, -1), "bf16")


def test_bwd_d256_long_causal():
    """d = 256 (two dK/dV passes): a slice of the long-causal-d256 shape,
    2 heads at N = 4096."""
    q, k, v, do = make(1, 2, 4096, 256, "bf16", seed=43)
    scale = 1.0 / 16
    grads, _, _ = run_bwd(q, k, v, do, scale, True)
    check(grads, q, k, v, do, scale, True, (-1, -1), "bf16")


def test_delta_is_rowsum_of_do_times_o():
    q, k, v, do = make(2, 3, 333, 128, "f16", seed=9)
    _, o, delta = run_bwd(q, k, v, do, 0.1, False)
    want = (do.double() * o.double()).sum(-1)
    assert (delta.double() - want).abs().max().item() <= 1e-4 * max(1.0, want.abs().max().item())


def test_zero_width_window_gradients():
    """window (0, 0): O = V, so dV = dO and dQ = dK = 0. P recomputes to 1
    within 1e-7, which rounds to exactly 1 in bf16, so dV = dO bit for bit;
    dQ and dK are fp32 rounding noise of dP - delta (both equal dO . V)."""
    q, k, v, do = make(1, 2, 300, 64, "bf16", seed=4)
    (dq, dk, dv), _, _ = run_bwd(q, k, v, do, 0.125, False, (0, 0))
    assert torch.equal(dv, do)
    assert dq.abs().max().item() <= 1e-5 and dk.abs().max().item() <= 1e-5


def test_bwd_deterministic():
    q, k, v, do = make(1, 4, 700, 128, "bf16", seed=12)
    a, _, _ = run_bwd(q, k, v, do, 0.09, True)
    b, _, _ = run_bwd(q, k, v, do, 0.09, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_matches_bwd():
    q, k, v, do = make(1, 2, 200, 64, "f16", seed=21)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qd, kd, vd, causal=True)
    o.backward(do.cuda())
    grads, _, _ = run_bwd(q, k, v, do, 1.0 / math.sqrt(64), True)
    for t, g in zip((qd, kd, vd), grads):
        assert torch.equal(t.grad.cpu(), g)


def test_bwd_python_errors():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device="cuda")
    lse = torch.zeros(1, 1, 8, device="cuda")
    with pytest.raises(NotImplementedError):
        fa.bwd(x, x, x, x, lse, x)
    y = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        fa.bwd(y, y, y, y, lse, y)
