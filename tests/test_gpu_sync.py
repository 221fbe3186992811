"""Race check: libfa.so against libfa_sync.so, the same sources built with
FA_SYNC_CHECK, where every wait drains all tile copies and every barrier is a
full one. The arithmetic is the same, so every output must be bitwise equal;
a wait or barrier missing in the normal build (a copy read before it landed,
a stage overwritten while another wave still reads it) would make the
results differ. Both libraries are called through their C ABI on the same
inputs, for the forward (plain, causal, window, split-KV, fewer queries than
keys, fp32) and the backward."""

import ctypes
import math
import sys

import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs

pytestmark = pytest.mark.gpu

VP = ctypes.c_void_p
I = ctypes.c_int


def load(path):
    lib = ctypes.CDLL(path)
    lib.fa_fwd_kv.restype = I
    lib.fa_fwd_kv.argtypes = [VP] * 5 + [VP, VP, ctypes.c_longlong, I] + [I] * 5 + [ctypes.c_float] + [I] * 4 + [VP]
    lib.fa_bwd_strided.restype = I
    lib.fa_bwd_strided.argtypes = [VP] * 11 + [I] * 4 + [ctypes.c_float] + [I] * 4 + [VP]
    return lib


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not fabuild.is_built():
        fabuild.build()
    return load(fabuild.LIB_PATH), load(fabuild.SYNC_LIB_PATH)


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()


CODE = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}


def fwd_with(lib, q, k, v, causal, window=(-1, -1), splits=1):
    B, H, N, D = q.shape
    Nk = k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    ws = torch.empty(max(fa.splitkv_workspace_bytes(B, H, N, D, max(splits, 1)), 16), dtype=torch.uint8, device="cuda")
    st = lib.fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), None,
                       ws.data_ptr(), ws.numel(), splits, B, H, N, Nk, D, 1.0 / math.sqrt(D), int(causal),
                       window[0], window[1], CODE[q.dtype], torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.strerror(st)
    torch.cuda.synchronize()
    return o, lse


FWD_CASES = [
    # (B, H, N, Nk, D, dtype, causal, window, splits)
    (1, 4, 2048, 2048, 256, "bf16", True, (-1, -1), 1),
    (1, 8, 1500, 1500, 128, "f16", False, (-1, -1), 1),
    (2, 3, 777, 777, 64, "bf16", True, (-1, -1), 1),
    (1, 2, 3000, 3000, 128, "bf16", True, (300, -1), 1),
    (1, 2, 4096, 4096, 128, "bf16", True, (-1, -1), 4),
    (1, 8, 1, 20000, 128, "bf16", True, (-1, -1), 8),
    (2, 2, 100, 2600, 256, "f16", False, (-1, -1), 1),
    (2, 2, 1000, 1000, 64, "f32", True, (-1, -1), 1),
]


@pytest.mark.parametrize("B,H,N,Nk,D,dtype,causal,window,splits", FWD_CASES)
def test_forward_matches_sync_build(libs, B, H, N, Nk, D, dtype, causal, window, splits):
    fast, sync = libs
    q = inputs.make_qkv(B, H, N, D, dtype, seed=N + D)[0].cuda()
    _, k, v = (t.cuda() for t in inputs.make_qkv(B, H, Nk, D, dtype, seed=Nk + 1))
    o1, l1 = fwd_with(fast, q, k, v, causal, window, splits)
    o2, l2 = fwd_with(sync, q, k, v, causal, window, splits)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o1).all()


def bwd_with(lib, q, k, v, o, lse, do, causal, window=(-1, -1)):
    B, H, N, D = q.shape
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.empty((B, H, N), device="cuda")
    st = lib.fa_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), None, B, H, N, D,
                            1.0 / math.sqrt(D), int(causal), window[0], window[1], CODE[q.dtype],
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.strerror(st)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("B,H,N,D,dtype,causal,window", [
    (1, 4, 2048, 128, "bf16", True, (-1, -1)),
    (2, 2, 999, 64, "f16", False, (-1, -1)),
    (1, 2, 1500, 256, "bf16", True, (-1, -1)),
    (1, 2, 1200, 128, "bf16", False, (100, 30)),
])
def test_backward_matches_sync_build(libs, B, H, N, D, dtype, causal, window):
    fast, sync = libs
    q, k, v = (t.cuda() for t in inputs.make_qkv(B, H, N, D, dtype, seed=N))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(N)).to(q.dtype).cuda()
    o, lse = fa.fwd(q, k, v, causal=causal, window_size=window)
    a = bwd_with(fast, q, k, v, o, lse, do, causal, window)
    b = bwd_with(sync, q, k, v, o, lse, do, causal, window)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
        assert torch.isfinite(x).all()
