"""GPU parity where element offsets pass 2^31.

One [B, H, 1024, 256] bf16 tensor of 8200 heads is 4.3 GB: head 8192 starts
at element 2^31 (byte 2^32), and the fp32 [1, 32800, 1024, 64] tensor does
the same at head 32768. The heads repeat a seeded pool of 67 distinct heads,
so a head read through an offset that wrapped at 2^32 bytes (head h - 8192,
or h - 32768) would hold another pool head's values and fail. The heads on
both sides of the boundary and the last head are checked row by row against
the fp64 oracle, for the head term of the offset (B = 1, many heads) in the
forward and for the batch term (many batches, H = 1) in the backward. The
tolerances are the parity tests' ones.
"""

import sys

import numpy as np
import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs
from oracle import attention_bwd_ref, attention_ref

pytestmark = pytest.mark.gpu

PERIOD = 67  # prime: no multiple of it is a power of two


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
    yield
    torch.cuda.empty_cache()


def heads64(t, heads):
    """Flat heads ``heads`` of a [B, H, N, D] tensor as a float64 array [1, len, N, D]."""
    flat = t.reshape(-1, *t.shape[2:])
    return flat[heads].to("cpu", torch.float64).numpy()[None]


@pytest.mark.parametrize("dtype,H,D,tol", [("bf16", 8200, 256, 1e-2), ("f32", 32800, 64, 1e-5)])
def test_forward_past_2_31_elements(dtype, H, D, tol):
    N = 1024
    assert H * N * D > 2 ** 31 and (2 ** 31) % (N * D) == 0
    q, k, v = inputs.make_cycled_heads(1, H, N, D, dtype, PERIOD, seed=31, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, H, N), float("nan"), dtype=torch.float32, device="cuda")
    scale = D ** -0.5
    fa.fwd(q, k, v, softmax_scale=scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    b = 2 ** 31 // (N * D)  # first head past the boundary
    heads = [b - 1, b, b + 1, H - 1]
    assert len({h % PERIOD for h in heads} | {(h - b) % PERIOD for h in heads[1:]}) == 7
    o_ref, lse_ref = attention_ref(heads64(q, heads), heads64(k, heads), heads64(v, heads), scale, True)
    err_o = np.abs(heads64(o, heads) - o_ref).max()
    err_l = np.abs(lse.reshape(H, N)[heads].cpu().double().numpy()[None] - lse_ref).max()
    assert err_o <= tol, f"max|dO| = {err_o:.3e}"
    assert err_l <= 1e-3, f"max|dLSE| = {err_l:.3e}"
    assert torch.isfinite(o[0, -1]).all() and torch.isfinite(lse).all()


def test_backward_past_2_31_elements():
    B, N, D = 8200, 1024, 256
    q, k, v = inputs.make_cycled_heads(B, 1, N, D, "bf16", PERIOD, seed=32, device="cuda")
    do = inputs.make_cycled_heads(B, 1, N, D, "bf16", PERIOD, seed=33, device="cuda")[0]
    scale = D ** -0.5
    o, lse = fa.fwd(q, k, v, softmax_scale=scale, causal=True)
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.bwd(q, k, v, o, lse, do, softmax_scale=scale, causal=True, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    b = 2 ** 31 // (N * D)
    heads = [b - 1, b, B - 1]
    ref = attention_bwd_ref(heads64(q, heads), heads64(k, heads), heads64(v, heads), heads64(do, heads), scale,
                            True)
    for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
        g = heads64(got, heads)
        assert np.isfinite(g).all(), f"{name}: unwritten or non-finite"
        err = np.abs(g - r).max() / max(np.abs(r).max(), 1.0)
        assert err <= 1e-2, f"{name}: max|d| / max(max|ref|, 1) = {err:.3e}"
