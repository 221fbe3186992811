"""GPU tests of strided operands: the head slices of packed tensors read and
written in place (fa_fwd_strided / fa_bwd_strided through the Python layer).

Two bars. Parity: the outputs against the fp64 oracle (forward: the bounds
of test_gpu_parity.py; backward: those of test_gpu_bwd.py), with the oracle
fed contiguous copies of the same values. Layout independence: the kernels
do the same arithmetic whatever the strides, so the strided results must be
bitwise equal to those of the contiguous call on copies of the inputs.
Outputs and their neighbours are pre-filled with NaN, so a missed or stray
write shows up.
"""

import math
import sys

import numpy as np
import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs
from oracle import attention_bwd_ref, attention_ref

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1e-2, torch.float32: 1e-5}
TOL_LSE = 1e-3
TOL_G = {torch.float16: 2e-3, torch.bfloat16: 1e-2}


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


def slices(qkv):
    """q, k, v of a packed [B, N, 3, H, d] tensor as [B, H, N, d] views."""
    return [qkv[:, :, i].transpose(1, 2) for i in range(3)]


def check_oracle(o, lse, q, k, v, scale, causal, window=(-1, -1)):
    o_ref, lse_ref = attention_ref(np64(q), np64(k), np64(v), scale, causal, window=window)
    err_o = np.abs(np64(o) - o_ref).max()
    err_l = np.abs(np64(lse) - lse_ref).max()
    assert err_o <= TOL_O[q.dtype], err_o
    assert err_l <= TOL_LSE, err_l


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_forward(dtype, D, causal):
    B, N, H = 2, 300, 3
    qkv = inputs.make_packed_qkv(B, N, H, D, dtype, seed=D + causal).cuda()
    scale = 1.0 / math.sqrt(D)
    o = fa.flash_attn_qkvpacked_func(qkv, causal=causal)
    assert o.shape == (B, N, H, D) and o.is_contiguous()
    # the same call on contiguous copies: bitwise equal
    qc, kc, vc = (t.contiguous() for t in slices(qkv))
    o_ref, lse_ref = fa.fwd(qc, kc, vc, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2), o_ref)
    _, lse = fa.fwd(*slices(qkv), causal=causal)
    assert torch.equal(lse, lse_ref)
    check_oracle(o.transpose(1, 2).cpu(), lse.cpu(), qc.cpu(), kc.cpu(), vc.cpu(), scale, causal)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bnhd_forward_and_strided_output(dtype):
    """q, k, v as [B, N, H, d] tensors; o written into slot 1 of a
    [B, N, 3, H, d] buffer whose other slots must stay untouched."""
    B, N, H, D = 2, 257, 4, 128
    q, k, v = (inputs.make_qkv(B, N, H, D, dtype, seed=s)[0].cuda() for s in (1, 2, 3))  # [B, N, H, D]
    big = torch.full((B, N, 3, H, D), float("nan"), dtype=DT[dtype], device="cuda")
    out = big[:, :, 1].transpose(1, 2)
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fwd(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), causal=True, out=out, lse=lse)
    o_ref, lse_ref = fa.fwd(*(t.transpose(1, 2).contiguous() for t in (q, k, v)), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, lse_ref)
    assert torch.isnan(big[:, :, 0]).all() and torch.isnan(big[:, :, 2]).all()
    o2 = fa.flash_attn_func(q, k, v, causal=True)
    assert o2.shape == (B, N, H, D) and torch.equal(o2.transpose(1, 2), o_ref)


def test_head_broadcast_kv():
    """A head stride of 0 shares one K and V among all heads."""
    B, H, N, D = 2, 5, 200, 64
    q, _, _ = inputs.make_qkv(B, H, N, D, "f16", seed=9)
    _, k1, v1 = inputs.make_qkv(B, 1, N, D, "f16", seed=10)
    qd, k1d, v1d = q.cuda(), k1.cuda(), v1.cuda()
    ke, ve = k1d.expand(B, H, N, D), v1d.expand(B, H, N, D)
    assert ke.stride(1) == 0
    o, lse = fa.fwd(qd, ke, ve)
    o_ref, lse_ref = fa.fwd(qd, ke.contiguous(), ve.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    check_oracle(o.cpu(), lse.cpu(), q, ke.contiguous().cpu(), ve.contiguous().cpu(), 1 / 8, False)


@pytest.mark.parametrize("window", [(40, 7), (100, -1)])
def test_packed_forward_window(window):
    B, N, H, D = 1, 513, 2, 128
    qkv = inputs.make_packed_qkv(B, N, H, D, "bf16", seed=31).cuda()
    _, lse = fa.fwd(*slices(qkv), window_size=window)
    o = fa.flash_attn_qkvpacked_func(qkv, window_size=window)
    o_ref, lse_ref = fa.fwd(*(t.contiguous() for t in slices(qkv)), window_size=window)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2), o_ref) and torch.equal(lse, lse_ref)


# ------------------------------------------------------------- backward --

def grads_contiguous(q, k, v, do, causal, window=(-1, -1)):
    o, lse = fa.fwd(q, k, v, causal=causal, window_size=window)
    return fa.bwd(q, k, v, o, lse, do, causal=causal, window_size=window)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_backward(dtype, D, causal):
    """flash_attn_qkvpacked_func's backward writes the packed gradient in
    place; it equals the contiguous backward bitwise and the oracle within
    the backward's bar."""
    B, N, H = 2, 333, 3
    qkv = inputs.make_packed_qkv(B, N, H, D, dtype, seed=5 * D + causal).cuda().requires_grad_(True)
    g = torch.Generator().manual_seed(77)
    do = torch.randn(B, N, H, D, generator=g).to(DT[dtype]).cuda()
    o = fa.flash_attn_qkvpacked_func(qkv, causal=causal)
    o.backward(do)
    dqkv = qkv.grad
    assert dqkv.shape == qkv.shape and dqkv.is_contiguous()
    qc, kc, vc = (t.detach().contiguous() for t in slices(qkv))
    dq, dk, dv = grads_contiguous(qc, kc, vc, do.transpose(1, 2).contiguous(), causal)
    torch.cuda.synchronize()
    for i, ref in enumerate((dq, dk, dv)):
        assert torch.equal(dqkv[:, :, i].transpose(1, 2), ref), f"slot {i}"
    want = attention_bwd_ref(np64(qc), np64(kc), np64(vc), np64(do.transpose(1, 2)), 1.0 / math.sqrt(D), causal)
    for got, ref in zip((dq, dk, dv), want):
        err = np.abs(np64(got) - ref).max() / max(np.abs(ref).max(), 1.0)
        assert err <= TOL_G[DT[dtype]], err


def test_bnhd_autograd_and_strided_gradients():
    """flash_attn_func on [B, N, H, d] views of one packed tensor: autograd
    accumulates the three [B, N, H, d] gradients into the packed leaf."""
    B, N, H, D = 1, 190, 4, 64
    leaf = inputs.make_packed_qkv(B, N, H, D, "bf16", seed=8).cuda().requires_grad_(True)
    q, k, v = (leaf[:, :, i] for i in range(3))
    g = torch.Generator().manual_seed(3)
    do = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16).cuda()
    fa.flash_attn_func(q, k, v, causal=True).backward(do)
    qc, kc, vc = (t.detach().transpose(1, 2).contiguous() for t in (q, k, v))
    ref = grads_contiguous(qc, kc, vc, do.transpose(1, 2).contiguous(), True)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(leaf.grad[:, :, i].transpose(1, 2), ref[i])


def test_strided_gradient_outputs_leave_neighbours():
    """dq, dk, dv written into slots 0, 2, 3 of a NaN-filled [B, N, 4, H, d]
    buffer; slot 1 stays NaN."""
    B, N, H, D = 2, 100, 2, 128
    q, k, v = (t.cuda() for t in inputs.make_qkv(B, H, N, D, "f16", seed=4))
    do = torch.randn(B, H, N, D, generator=torch.Generator().manual_seed(5)).half().cuda()
    o, lse = fa.fwd(q, k, v)
    buf = torch.full((B, N, 4, H, D), float("nan"), dtype=torch.float16, device="cuda")
    views = [buf[:, :, s].transpose(1, 2) for s in (0, 2, 3)]
    fa.bwd(q, k, v, o, lse, do, dq=views[0], dk=views[1], dv=views[2])
    ref = fa.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for got, want in zip(views, ref):
        assert torch.equal(got, want)
    assert torch.isnan(buf[:, :, 1]).all()


def test_python_layer_rejects_overlapping_output():
    qkv = inputs.make_packed_qkv(1, 64, 2, 64, "f16").cuda()
    q, k, v = slices(qkv)
    with pytest.raises(fa.FaError, match="FA_ERR_ARG"):
        fa.fwd(q, k, v, out=k)
    with pytest.raises(ValueError, match="last dimension"):
        fa.fwd(q, k, v.transpose(2, 3))
