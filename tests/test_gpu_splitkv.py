"""GPU parity of split-KV attention (fa_fwd_splitkv): the merged output
against the fp64 oracle (bounds of test_gpu_parity.py), and the partial
results the parts leave in the workspace against the oracle's partial
attention over the same key ranges (oracle/splitkv.py). Outputs are
pre-filled with NaN."""

import math
import sys

import numpy as np
import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs
from oracle import attention_ref
from oracle.splitkv import partial_ref

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1e-2, torch.float32: 1e-5}
TOL_LSE = 1e-3
CODE = {torch.float16: fa.FA_F16, torch.bfloat16: fa.FA_BF16, torch.float32: fa.FA_F32}


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


def run_split(q, k, v, causal, splits, window=(-1, -1), workspace=None):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(qd, kd, vd, causal=causal, window_size=window, out=o, lse=lse, num_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, q, k, v, causal, window=(-1, -1)):
    scale = 1.0 / math.sqrt(q.shape[-1])
    o_ref, lse_ref = attention_ref(np64(q), np64(k), np64(v), scale, causal, window=window)
    assert np.isfinite(np64(o)).all() and np.isfinite(np64(lse)).all()
    err_o = np.abs(np64(o) - o_ref).max()
    err_l = np.abs(np64(lse) - lse_ref).max()
    assert err_o <= TOL_O[q.dtype], err_o
    assert err_l <= TOL_LSE, err_l


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [2, 5])
def test_split_parity(dtype, D, causal, splits):
    q, k, v = inputs.make_qkv(2, 2, 333, D, dtype, seed=D + splits)
    o, lse = run_split(q, k, v, causal, splits)
    check(o, lse, q, k, v, causal)


@pytest.mark.parametrize("N,splits", [(1, 3), (64, 4), (100, 7), (129, 64)])
def test_more_parts_than_tiles(N, splits):
    """Parts with no key tile (n < S) write O_s = 0, LSE_s = -inf and weigh 0."""
    q, k, v = inputs.make_qkv(1, 3, N, 128, "bf16", seed=N)
    for causal in (False, True):
        o, lse = run_split(q, k, v, causal, splits)
        check(o, lse, q, k, v, causal)


@pytest.mark.parametrize("window", [(0, 0), (17, 5), (200, -1), (-1, 33)])
def test_split_window(window):
    """Windows leave rows with no visible key in some parts."""
    q, k, v = inputs.make_qkv(1, 2, 700, 64, "f16", seed=7)
    o, lse = run_split(q, k, v, False, 6, window)
    check(o, lse, q, k, v, False, window)


def tile_ranges(N, rows_per_tile, causal, window, S, s):
    """Per-row key range [lo, hi) of part s: the documented partition of each
    query tile's key tiles (64 keys each)."""
    left, right = window
    if causal:
        right = 0
    lo = np.zeros(N, np.int64)
    hi = np.zeros(N, np.int64)
    for t0 in range(0, N, rows_per_tile):
        q_last = min(t0 + rows_per_tile - 1, N - 1)
        first = max(t0 - left, 0) // 64 if left >= 0 else 0
        last = min(q_last + right, N - 1) // 64 if right >= 0 else (N - 1) // 64
        n = last + 1 - first
        a, e = first + n * s // S, first + n * (s + 1) // S
        lo[t0:q_last + 1] = a * 64
        hi[t0:q_last + 1] = min(e * 64, N)
    return lo, hi


@pytest.mark.parametrize("dtype,causal,window", [("bf16", True, (-1, -1)), ("f32", False, (90, 20)),
                                                 ("f16", False, (-1, -1))])
def test_workspace_partials(dtype, causal, window):
    """The parts' O_s and LSE_s in the workspace match the oracle's partial
    attention over each part's key range."""
    B, H, N, D, S = 1, 2, 300, 64, 3
    q, k, v = inputs.make_qkv(B, H, N, D, dtype, seed=11)
    ws = torch.full((fa.splitkv_workspace_bytes(B, H, N, D, S) // 4,), float("nan"), device="cuda")
    run_split(q, k, v, causal, S, window, workspace=ws)
    w = ws.cpu().numpy().astype(np.float64)
    o_parts = w[:S * B * H * N * D].reshape(S, B, H, N, D)
    l_parts = w[S * B * H * N * D:].reshape(S, B, H, N)
    rows = fa.grid(B, H, N, D, causal, CODE[q.dtype])[1]
    scale = 1.0 / math.sqrt(D)
    for s in range(S):
        lo, hi = tile_ranges(N, rows, causal, window, S, s)
        o_ref, l_ref = partial_ref(np64(q), np64(k), np64(v), scale, causal, lo, hi, window)
        empty = np.isneginf(l_ref)
        assert (np.isneginf(l_parts[s]) == empty).all(), f"part {s}: -inf rows differ"
        assert (o_parts[s][empty] == 0).all()
        # O_s is fp32 from rounded inputs: the forward's bound for the type
        assert np.abs(o_parts[s] - o_ref).max() <= TOL_O[q.dtype], s
        assert np.abs(l_parts[s][~empty] - l_ref[~empty]).max() <= TOL_LSE, s


def test_auto_and_single_split():
    # num_splits=1 is the plain kernel (bitwise); num_splits=0 lets the library choose
    q, k, v = inputs.make_qkv(1, 1, 4096, 128, "bf16", seed=3)
    o1, l1 = run_split(q, k, v, True, 1)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o_ref, l_ref = fa.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o_ref.cpu()) and torch.equal(l1, l_ref.cpu())
    assert fa.splitkv_num_splits(1, 1, 4096, 128, True) > 1
    o0, l0 = run_split(q, k, v, True, 0)
    check(o0, l0, q, k, v, True)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_configs_split(cfg):
    c = inputs.CONFIGS[cfg]
    q, k, v = inputs.make_config(cfg)
    for splits in (0, 2, 4):
        o, lse = run_split(q, k, v, c["causal"], splits)
        check(o, lse, q, k, v, c["causal"])


def test_strided_split_and_workspace_reuse():
    """Packed inputs with split-KV; one workspace for two calls, the second
    smaller."""
    qkv = inputs.make_packed_qkv(1, 500, 3, 128, "bf16", seed=2).cuda()
    sl = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
    ws = torch.empty(fa.splitkv_workspace_bytes(1, 3, 500, 128, 4), dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(*sl, causal=True, num_splits=4, workspace=ws)
    o2, lse2 = fa.fwd(*(t[:, :, :200] for t in sl), causal=True, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    qc, kc, vc = (t.contiguous().cpu() for t in sl)
    check(o.cpu(), lse.cpu(), qc, kc, vc, True)
    check(o2.cpu(), lse2.cpu(), *(t[:, :, :200].contiguous() for t in (qc, kc, vc)), True)


def test_workspace_errors():
    q = torch.zeros(1, 1, 256, 64, dtype=torch.float16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaError, match="FA_ERR_ARG"):
        fa.fwd(q, q, q, num_splits=2, workspace=small)
    with pytest.raises(fa.FaError, match="FA_ERR_ARG"):
        fa.fwd(q, q, q, num_splits=65)
