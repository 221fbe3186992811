"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (fixed for this method): max |O - O_oracle| <= 2e-3 for fp16 inputs,
1e-2 for bf16, 1e-5 for fp32; max |LSE - LSE_oracle| <= 1e-3. The five
workloads are held to that bar as stated; the other cases per element to
that bar or, where it is larger, to the worst case of the 16-bit roundings
for that element (``check``). The oracle sees
exactly the stored (rounded) inputs, so input quantisation is not counted.
Outputs are pre-filled with NaN so an element the kernel fails to write
shows up as a failure.
"""

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
U16 = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}  # unit roundoff of the 16-bit input types
DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


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


def run(q, k, v, scale, causal, window=(-1, -1)):
    """q, k, v: CPU tensors. Returns CPU (o, lse) from the HIP kernels."""
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(qd, kd, vd, softmax_scale=scale, causal=causal, window_size=window, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, q, k, v, scale, causal, rows=None, tol_o=None, window=(-1, -1), stated=False):
    """O and LSE against the oracle. O: the stated tolerance of the input
    type per element or, where it is larger, the worst case of the 16-bit
    path's two roundings for that element, u (A_ic + |O_ic|) with A the
    attention of the same scores over |V| and u the unit roundoff of the
    input type (2^-8 bf16, 2^-11 fp16). That second term exceeds the stated
    bound only in rows whose softmax sits on a few keys (narrow windows,
    the first rows of a causal or windowed sequence), where |O| reaches 2-4
    and output rounding alone can pass 1e-2 in bf16. stated=True (the five
    workloads) applies the stated tolerance alone."""
    o_ref, lse_ref = attention_ref(np64(q), np64(k), np64(v), scale, causal, rows=rows, window=window)
    o64, l64 = np64(o), np64(lse)
    if rows is not None:
        o64, l64 = o64[:, :, rows], l64[:, :, rows]
    assert np.isfinite(o64).all() and np.isfinite(l64).all(), "unwritten or non-finite output"
    err = np.abs(o64 - o_ref)
    err_l = np.abs(l64 - lse_ref).max()
    tol = TOL_O[q.dtype] if tol_o is None else tol_o
    bound = tol
    if not stated and q.dtype in U16:
        a_abs, _ = attention_ref(np64(q), np64(k), np.abs(np64(v)), scale, causal, rows=rows, window=window)
        bound = np.maximum(tol, U16[q.dtype] * (a_abs + np.abs(o_ref)))
    assert (err <= bound).all(), f"max|dO| = {err.max():.3e}, worst ratio to the bound {(err / bound).max():.3f}"
    assert err_l <= TOL_LSE, f"max|dLSE| = {err_l:.3e} > {TOL_LSE:.1e}"
    return err.max(), err_l


# ------------------------------------------------------------ the configs --

@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_full(cfg):
    c = inputs.CONFIGS[cfg]
    q, k, v = inputs.make_config(cfg)
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = run(q, k, v, scale, c["causal"])
    check(o, lse, q, k, v, scale, c["causal"], stated=True)


def test_config2_packed_entry():
    """The packed call reads the slices of qkv in place; o is [B, N, H, d]."""
    c = inputs.CONFIGS[2]
    qkv = inputs.make_packed_qkv(c["B"], c["N"], c["H"], c["D"], c["dtype"])
    qkvd = qkv.cuda()
    o = fa.flash_attn_qkvpacked_func(qkvd, dropout_p=0.0, softmax_scale=None, causal=False)
    assert o.shape == (c["B"], c["N"], c["H"], c["D"])
    _, lse = fa.fwd(*(qkvd[:, :, i].transpose(1, 2) for i in range(3)))
    torch.cuda.synchronize()
    q, k, v = inputs.unpack_qkv(qkv)
    check(o.transpose(1, 2).cpu(), lse.cpu(), q, k, v, 1.0 / math.sqrt(c["D"]), False, stated=True)


def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    head = np.arange(min(N, 256))
    tail = np.arange(max(0, N - 64), N)
    mid = rng.choice(N, size=min(N, 96), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


@pytest.mark.parametrize("cfg", [4, 5])
def test_config_large_all_rows(cfg):
    """Full-size launch; every row of every head against the oracle (the
    long-sequence workload's oracle takes about half a minute on 16 cores)."""
    c = inputs.CONFIGS[cfg]
    q, k, v = inputs.make_config(cfg)
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = run(q, k, v, scale, c["causal"])
    check(o, lse, q, k, v, scale, c["causal"], stated=True)


# ---------------------------------------------------------------- edges --

EDGE_N = [1, 2, 17, 63, 64, 65, 100, 127, 128, 129, 257, 1000]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths(dtype, D, causal):
    for N in EDGE_N:
        q, k, v = inputs.make_qkv(1, 3, N, D, dtype, seed=N)
        scale = 1.0 / math.sqrt(D)
        o, lse = run(q, k, v, scale, causal)
        check(o, lse, q, k, v, scale, causal)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_batch_heads_and_long_ragged(dtype):
    q, k, v = inputs.make_qkv(2, 5, 4097, 64, dtype, seed=7)
    for causal in (False, True):
        o, lse = run(q, k, v, 0.125, causal)
        check(o, lse, q, k, v, 0.125, causal, rows=_sample_rows(4097, 3))


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_other_scales(scale):
    """Scales other than 1/sqrt(d). In fp32 the rounding of the scores and of
    the exponent argument grows with the logit magnitude |scale| * |q||k|,
    so the fp32 bound 1e-5 (stated for scale 1/sqrt(d)) is widened by
    max(1, |scale| sqrt(d)), the ratio of the logit spread to the default's."""
    D = 128
    q, k, v = inputs.make_qkv(1, 2, 200, D, "f32", seed=11)
    tol = 1e-5 * max(1.0, abs(scale) * math.sqrt(D))
    for causal in (False, True):
        o, lse = run(q, k, v, scale, causal)
        check(o, lse, q, k, v, scale, causal, tol_o=tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_reference_moves_on_growing_logits(dtype, D):
    """Key norms that grow along the sequence (x0.05 .. x4) at twice the
    default scale make later key tiles' scores exceed the first tile's
    maximum by far more than 8 in exp2 units, the point at which the 16-bit
    kernel moves its exponent reference and rescales the output it has
    accumulated so far: many rows take that rare path, in tiles after
    the first. V is scaled by 1/4, so |O| stays below about 1 and the usual
    bound applies to the peaky softmax this gives."""
    N = 700
    q, k, v = inputs.make_qkv(1, 2, N, D, dtype, seed=21)
    ramp = torch.linspace(0.05, 4.0, N).view(1, 1, N, 1)
    k = (k.float() * ramp).to(k.dtype)
    v = (v.float() * 0.25).to(v.dtype)
    scale = 2.0 / math.sqrt(D)
    # The inputs do force moves: per row, the scores' maximum over all keys
    # minus their maximum over the first 64 keys, in exp2 units.
    s2 = np64(q)[0, 0] @ np64(k)[0, 0].T * scale * math.log2(math.e)
    assert ((s2.max(axis=1) - s2[:, :64].max(axis=1)) > 8).mean() > 0.9
    for causal in (False, True):
        o, lse = run(q, k, v, scale, causal)
        check(o, lse, q, k, v, scale, causal)
    o, lse = run(q, k, v, scale, True, window=(300, -1))
    check(o, lse, q, k, v, scale, True, window=(300, -1))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_reference_moves_on_growing_logits_f32(D):
    """The same growing-logit inputs in fp32. At d <= 128 the fp32 kernel keeps
    the lazy exponent reference too (the reference moves for a row whose P
    sum over a 32-key block exceeds 2^8), at d = 256 the exact running max.
    The stated fp32 bound applies (measured: at most 6e-6)."""
    N = 700
    q, k, v = inputs.make_qkv(1, 2, N, D, "f32", seed=21)
    ramp = torch.linspace(0.05, 4.0, N).view(1, 1, N, 1)
    k = k * ramp
    v = v * 0.25
    scale = 2.0 / math.sqrt(D)
    s2 = np64(q)[0, 0] @ np64(k)[0, 0].T * scale * math.log2(math.e)
    assert ((s2.max(axis=1) - s2[:, :32].max(axis=1)) > 8).mean() > 0.9
    for causal in (False, True):
        o, lse = run(q, k, v, scale, causal)
        check(o, lse, q, k, v, scale, causal)
    o, lse = run(q, k, v, scale, True, window=(300, -1))
    check(o, lse, q, k, v, scale, True, window=(300, -1))


# ----------------------------------------------------- GPU-side invariants --

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_identical_keys_and_zero_scale_give_means(dtype):
    N, D = 300, 128
    q, k, v = inputs.make_qkv(1, 1, N, D, dtype, seed=5)
    k = k[:, :, :1].expand(1, 1, N, D).contiguous()
    tol = TOL_O[DT[dtype]]
    for causal in (False, True):
        o, _ = run(q, k, v, 1.0 / math.sqrt(D), causal)
        v64 = np64(v)[0, 0]
        want = np.cumsum(v64, 0) / np.arange(1, N + 1)[:, None] if causal else v64.mean(0)[None]
        assert np.abs(np64(o)[0, 0] - want).max() <= tol
        o0, lse0 = run(q, k, v, 0.0, causal)
        assert np.abs(np64(o0)[0, 0] - want).max() <= tol
        counts = np.arange(1, N + 1) if causal else np.full(N, N)
        assert np.abs(np64(lse0)[0, 0] - np.log(counts)).max() <= TOL_LSE


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_single_key_and_causal_first_row(dtype):
    q, k, v = inputs.make_qkv(2, 3, 1, 64, dtype, seed=9)
    o, lse = run(q, k, v, 0.125, False)
    assert torch.equal(o, v)
    q, k, v = inputs.make_qkv(1, 2, 500, 64, dtype, seed=10)
    o, _ = run(q, k, v, 0.125, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])


@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("f16", 128), ("f32", 64), ("bf16", 64)])
def test_causal_rows_ignore_later_keys(dtype, D):
    """Causal structure: changing the keys and values after row i0 leaves
    rows 0..i0 unchanged bit for bit, the rows of the query tile that holds
    i0 included (there the changed keys are loaded but masked, and the
    exponent reference of the 16-bit kernel moves per row, on that row's
    visible keys only); later rows change."""
    N, i0 = 700, 300
    q, k, v = inputs.make_qkv(1, 2, N, D, dtype, seed=14)
    o1, l1 = run(q, k, v, 0.1, True)
    k2, v2 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(15)
    k2[:, :, i0 + 1:] = torch.randn(k2[:, :, i0 + 1:].shape, generator=g).to(k.dtype) * 3
    v2[:, :, i0 + 1:] = torch.randn(v2[:, :, i0 + 1:].shape, generator=g).to(v.dtype) * 3
    o2, l2 = run(q, k2, v2, 0.1, True)
    assert torch.equal(o1[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    assert torch.equal(l1[:, :, :i0 + 1], l2[:, :, :i0 + 1])
    assert not torch.equal(o1[:, :, i0 + 1:], o2[:, :, i0 + 1:])


def test_constant_values():
    q, k, _ = inputs.make_qkv(1, 4, 777, 256, "bf16", seed=12)
    v = torch.full_like(q, 1.5)
    for causal in (False, True):
        o, _ = run(q, k, v, 0.0625, causal)
        assert torch.equal(o, v)


def test_grid_remap_does_not_change_results():
    """With a grid that is a multiple of 8 the workgroup -> (head, tile) map
    is permuted across XCDs; with 7 heads it is the identity. Heads 0..6
    come out bitwise the same either way."""
    q, k, v = inputs.make_qkv(1, 8, 1024, 128, "bf16", seed=16)
    o8, l8 = run(q, k, v, 0.088, True)       # 8 heads x 8 tiles = 64 workgroups (remapped)
    o7, l7 = run(q[:, :7].contiguous(), k[:, :7].contiguous(), v[:, :7].contiguous(), 0.088, True)  # 56: identity
    assert torch.equal(o8[:, :7], o7) and torch.equal(l8[:, :7], l7)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_length_4097_sampled_rows(dtype, D):
    """N = 4097: one row past a power of two, so the last query tile and the
    last key tile hold a single row."""
    q, k, v = inputs.make_qkv(1, 1, 4097, D, dtype, seed=D + 4097)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(4000, 4097), [1023, 1024, 2048]]))
    for causal in (False, True):
        o, lse = run(q, k, v, 1.0 / math.sqrt(D), causal)
        check(o, lse, q, k, v, 1.0 / math.sqrt(D), causal, rows=rows)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_deterministic_bitwise():
    q, k, v = inputs.make_qkv(1, 8, 1500, 128, "bf16", seed=13)
    outs = [run(q, k, v, 0.088, True) for _ in range(3)]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_zero_size_inputs():
    q = torch.empty(0, 2, 16, 64, dtype=torch.float16, device="cuda")
    o, lse = fa.fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.empty(1, 2, 0, 64, dtype=torch.float16, device="cuda")
    o, lse = fa.fwd(q, q, q)
    assert o.numel() == 0


def test_python_layer_errors():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.float16, device="cuda")
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q)
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float64, device="cuda")
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q)
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd(q, q, q.transpose(2, 3))


# ------------------------------------------------- local-attention window --

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_window_shapes(dtype, D, causal):
    """Windows narrower than a tile, straddling tiles, one-sided and wider
    than the sequence, on ragged lengths."""
    for N, window in ((257, (0, 0)), (257, (5, 3)), (300, (64, 0)), (300, (70, 129)),
                      (1000, (200, -1)), (1000, (-1, 33)), (129, (1000, 1000))):
        q, k, v = inputs.make_qkv(1, 2, N, D, dtype, seed=N + D + window[0])
        scale = 1.0 / math.sqrt(D)
        o, lse = run(q, k, v, scale, causal, window)
        check(o, lse, q, k, v, scale, causal, window=window)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_window_zero_width_returns_v_exactly(dtype):
    """window (0, 0): each row sees only its own key, so O = V bit for bit."""
    q, k, v = inputs.make_qkv(2, 3, 515, 128, dtype, seed=7)
    o, lse = run(q, k, v, 0.1, False, (0, 0))
    assert torch.equal(o, v)
    want = 0.1 * (q.double() * k.double()).sum(-1)
    assert (lse.double() - want).abs().max().item() <= 1e-3


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (256, "bf16"), (64, "f32")])
def test_window_long_sequence_sampled_rows(D, dtype):
    """A 4096-key causal sliding window of 512 on a long sequence: many full
    tiles in the middle, masked tiles at both ends of each block's range."""
    N = 8192 if dtype != "f32" else 4096
    q, k, v = inputs.make_qkv(1, 2, N, D, dtype, seed=11)
    rows = np.unique(np.concatenate([np.arange(200), np.arange(N // 2 - 100, N // 2 + 100), np.arange(N - 200, N)]))
    for causal, window in ((True, (512, -1)), (False, (300, 300))):
        o, lse = run(q, k, v, 1.0 / math.sqrt(D), causal, window)
        check(o, lse, q, k, v, 1.0 / math.sqrt(D), causal, rows=rows, window=window)


def test_window_minus_one_matches_plain_call():
    """window (-1, -1) goes through the same kernels as fa_fwd: identical bits."""
    q, k, v = inputs.make_qkv(1, 4, 777, 128, "bf16", seed=5)
    o1, l1 = run(q, k, v, 0.09, True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o2 = torch.empty_like(qd)
    l2 = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    st = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(), 1, 4, 777, 128,
                   0.09, 1, fa.FA_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.cpu()) and torch.equal(l1, l2.cpu())
