"""fa_fwd_kv_noalloc (the allocation-free split-KV forward, whose partial
results live in the library's static device array) against fa_fwd_kv with
a caller workspace, through the C ABI: the same kernels with the same parts
give bitwise the same O and LSE. Two calls in a row, the second with a
smaller input (the array keeps the first call's contents, which must not
matter), then a plain call (one part: no scratch) and a decode step."""

import math
import sys

import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs

pytestmark = pytest.mark.gpu

DT = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not fabuild.is_built():
        fabuild.build()
    fa.lib()


def both(B, H, N, Nk, D, dtype, causal, splits, seed):
    sys.__stderr__.write(f"\n[gpu case] noalloc B={B} H={H} N={N} Nk={Nk} d={D} {dtype} causal={causal} "
                         f"splits={splits}\n")
    sys.__stderr__.flush()
    q = inputs.make_qkv(B, H, N, D, dtype, seed=seed)[0].cuda()
    _, k, v = (t.cuda() for t in inputs.make_qkv(B, H, Nk, D, dtype, seed=seed + 1))
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream().cuda_stream
    ns = splits if splits else fa.splitkv_num_splits(B, H, N, D, causal, dtype=DT[dtype], Nk=Nk)
    nbytes = fa.splitkv_workspace_bytes(B, H, N, D, ns) if ns > 1 else 0
    assert nbytes <= fa.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    o1, o2 = (torch.full_like(q, float("nan")) for _ in range(2))
    l1, l2 = (torch.full((B, H, N), float("nan"), device="cuda") for _ in range(2))
    st = fa.fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(), None, ws.data_ptr(),
                      nbytes, splits, B, H, N, Nk, D, scale, int(causal), -1, -1, DT[dtype], stream)
    assert st == 0, fa.strerror(st)
    st = fa.fa_fwd_kv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), None, splits,
                              B, H, N, Nk, D, scale, int(causal), -1, -1, DT[dtype], stream)
    assert st == 0, fa.strerror(st)
    torch.cuda.synchronize()
    assert torch.isfinite(o2).all() and torch.isfinite(l2).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    return ns


def test_noalloc_matches_workspace_call_twice_then_smaller():
    ns = both(1, 8, 200, 3000, 128, "bf16", True, 0, seed=1)     # library's choice of parts
    assert ns > 1
    ns = both(1, 2, 70, 900, 64, "f16", False, 3, seed=2)         # smaller input, 3 parts
    assert ns == 3


def test_noalloc_plain_and_decode():
    assert both(1, 3, 130, 130, 256, "bf16", True, 1, seed=3) == 1  # one part: no scratch
    assert both(1, 32, 1, 32768, 128, "bf16", True, 0, seed=4) > 1  # decode step
    both(2, 2, 33, 500, 64, "f32", False, 4, seed=5)


def test_noalloc_rejects_oversized_partials():
    q = torch.zeros(1, 64, 1024, 256, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 64, 1024, device="cuda")
    st = fa.fa_fwd_kv_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(), None, 2,
                              1, 64, 1024, 1024, 256, 0.0625, 1, -1, -1, fa.FA_BF16,
                              torch.cuda.current_stream().cuda_stream)
    assert st == -8
