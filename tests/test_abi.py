"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.
No test here launches a kernel (no GPU is needed)."""

import ctypes
import os
import re

import pytest

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not fabuild.is_built():
        fabuild.build()
    return fa.lib()


def declared_functions():
    with open(os.path.join(ROOT, "include", "fa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == sorted(fa.EXPORTS)
    for name in names:
        assert hasattr(fa.lib(), name), name


def test_strerror_covers_codes():
    for code in list(fa.STATUS) + [12345]:
        assert fa.strerror(code)
    assert "head dimension" in fa.strerror(-3)


GOOD = dict(q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=0x5000, B=1, H=2, N=100, d=64,
            scale=0.125, causal=0, dtype=1)


def call(**kw):
    a = dict(GOOD, **kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                     a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(H=-3), -2), (dict(N=-1), -2), (dict(d=-64), -2),
    (dict(N=1 << 30), -2), (dict(B=1 << 20, H=1 << 20, N=1 << 10), -2),
    (dict(d=32), -3), (dict(d=96), -3), (dict(d=512), -3),
    (dict(dtype=3), -4), (dict(dtype=-1), -4),
    (dict(causal=2), -6), (dict(causal=-1), -6),
    (dict(scale=float("nan")), -6), (dict(scale=float("inf")), -6),
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1), (dict(lse=0), -1),
    (dict(q=0x1008), -5), (dict(o=0x4004), -5), (dict(lse=0x5002), -5),
    (dict(o=0x1000), -6), (dict(lse=0x3000 + 64), -6), (dict(o=0x4000, lse=0x4000 + 128), -6),
])
def test_validation_errors(kw, code):
    # every case fails a host-side check, so no HIP call is made
    assert call(**kw) == code


def call_window(left, right, **kw):
    a = dict(GOOD, **kw)
    return fa.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                            a["scale"], a["causal"], left, right, a["dtype"], None)


@pytest.mark.parametrize("left,right", [(-2, 0), (0, -2), (-5, -5), (-(1 << 31), 3)])
def test_window_sides_below_minus_one_rejected(left, right):
    assert call_window(left, right) == -6
    # checked before the zero-size early return, so also without a launch
    assert call_window(left, right, N=0, q=0, k=0, v=0, o=0, lse=0) == -6


@pytest.mark.parametrize("kw,code", [(dict(d=96), -3), (dict(causal=2), -6), (dict(q=0), -1)])
def test_window_entry_shares_the_checks(kw, code):
    assert call_window(3, 0, **kw) == code


def test_python_window_argument_checked():
    with pytest.raises(ValueError):
        fa._window((-2, 0))
    with pytest.raises(ValueError):
        fa._window(5)
    assert fa._window((3, -1)) == (3, -1)


BWD = dict(q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=0x5000, do=0x6000, dq=0x10000, dk=0x20000,
           dv=0x30000, delta=0x40000, B=1, H=1, N=16, d=64, scale=0.125, causal=0, wl=-1, wr=-1, dtype=1)


def call_bwd(**kw):
    a = dict(BWD, **kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                     a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["wl"], a["wr"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(N=1 << 30), -2),
    (dict(d=512), -3), (dict(d=32), -3),
    (dict(dtype=2), -4), (dict(dtype=7), -4),
    (dict(causal=3), -6), (dict(scale=float("nan")), -6), (dict(wl=-2), -6),
    (dict(q=0), -1), (dict(do=0), -1), (dict(delta=0), -1), (dict(dv=0), -1),
    (dict(dq=0x10008), -5), (dict(delta=0x40002), -5),
    (dict(dq=0x1000), -6), (dict(dk=0x6000 + 32), -6), (dict(delta=0x5000), -6), (dict(dv=0x20000 + 64), -6),
])
def test_bwd_validation_errors(kw, code):
    # every case fails a host-side check, so no HIP call is made
    assert call_bwd(**kw) == code


def test_bwd_zero_size_is_a_noop():
    assert call_bwd(N=0, q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, delta=0) == 0


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_zero_size_is_a_noop(kw):
    # no launch and no pointer checks when there is nothing to compute
    assert call(q=0, k=0, v=0, o=0, lse=0, **kw) == 0


def test_grid_query():
    assert fa.grid(1, 16, 16384, 256, 1, 1) == (16 * 128, 128)
    assert fa.grid(2, 12, 256, 64, 0, 0) == (24 * 2, 128)
    assert fa.grid(1, 1, 1, 64, 0, 2) == (1, 64)
    assert fa.grid(4, 1, 4096, 64, 0, 2) == (4 * 64, 64)
    # causal 16-bit d = 64: query tiles nqt - 1 - p and p share a workgroup
    assert fa.grid(1, 64, 4096, 64, 1, 1) == (64 * 16, 128)
    assert fa.grid(2, 3, 300, 64, 1, 0) == (6 * 2, 128)       # 3 tiles: pairs (2, 0) and (1, 1)
    assert fa.grid(1, 2, 100, 64, 1, 0) == (2, 128)           # a single tile: the plain grid
    assert fa.grid(1, 128, 2048, 128, 1, 1) == (128 * 16, 128)  # d = 128: the plain grid
    assert fa.grid(1, 64, 4096, 64, 1, 2) == (64 * 64, 64)     # fp32: the plain grid
    with pytest.raises(fa.FaError):
        fa.grid(1, 1, 1, 80, 0, 2)


def test_python_layer_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(q, q, q)
    with pytest.raises(NotImplementedError):
        fa.flash_attn_qkvpacked_func(torch.zeros(1, 8, 3, 1, 64), dropout_p=0.1)
