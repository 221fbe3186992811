"""HIP graph capture: the library's calls enqueue kernels only (no
allocation, no memset, no host synchronisation), so they can be captured
into a HIP graph (torch.cuda.graph) and replayed. Each test captures calls
with preallocated outputs, replays the graph several times with eager work
and synchronisations in between, and checks every replay against the eager
result bit for bit (inputs are changed between replays to show that each
replay recomputes)."""

import sys

import pytest
import torch

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild
from transformer_exact_attention_flashattention_amd import inputs

pytestmark = pytest.mark.gpu


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


def replay_and_check(graph, static_in, make_inputs, outs, eager):
    """For three fresh input sets: copy them into the captured buffers,
    replay, and compare the captured outputs with an eager call."""
    for seed in (101, 102, 103):
        new = make_inputs(seed)
        for dst, src in zip(static_in, new):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = eager(*new)
        torch.cuda.synchronize()
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref), f"replay with seed {seed} differs from the eager call"


@pytest.mark.parametrize("dtype,D,causal", [("bf16", 128, True), ("f16", 64, False), ("f32", 64, False)])
def test_forward_in_graph(dtype, D, causal):
    B, H, N = 2, 3, 700
    mk = lambda seed: [t.cuda() for t in inputs.make_qkv(B, H, N, D, dtype, seed=seed)]  # noqa: E731
    q, k, v = mk(100)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda")
    fa.fwd(q, k, v, causal=causal, out=o, lse=lse)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
    replay_and_check(g, (q, k, v), mk, (o, lse), lambda a, b, c: fa.fwd(a, b, c, causal=causal))


def test_splitkv_in_graph():
    """Two kernels per call (parts, then merge) with a caller workspace."""
    B, H, N, D = 1, 2, 3000, 128
    mk = lambda seed: [t.cuda() for t in inputs.make_qkv(B, H, N, D, "bf16", seed=seed)]  # noqa: E731
    q, k, v = mk(100)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda")
    ws = torch.empty(fa.splitkv_workspace_bytes(B, H, N, D, 4), dtype=torch.uint8, device="cuda")
    fa.fwd(q, k, v, causal=True, out=o, lse=lse, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse, num_splits=4, workspace=ws)
    replay_and_check(g, (q, k, v), mk, (o, lse),
                     lambda a, b, c: fa.fwd(a, b, c, causal=True, num_splits=4, workspace=ws))


def test_backward_in_graph():
    """Forward and backward (delta, dQ, dK/dV kernels) in one graph."""
    B, H, N, D = 1, 2, 600, 128

    def mk(seed):
        q, k, v = inputs.make_qkv(B, H, N, D, "bf16", seed=seed)
        g = torch.Generator().manual_seed(seed + 7)
        do = torch.randn(q.shape, generator=g).to(q.dtype)
        return [t.cuda() for t in (q, k, v, do)]

    q, k, v, do = mk(100)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), device="cuda")

    def step():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    def eager(a, b, c, e):
        oo, ll = fa.fwd(a, b, c, causal=True)
        return (oo, ll) + fa.bwd(a, b, c, oo, ll, e, causal=True)

    replay_and_check(g, (q, k, v, do), mk, (o, lse, dq, dk, dv), eager)
