"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of attention's arithmetic: it only draws numbers and
moves them into the [B, H, N, d] layout. Both the oracle's callers and the
HIP path's callers take their inputs from here, so the two sides see the
same bits.

Recipe (the pages' workloads are i.i.d. standard-normal tensors drawn after
``torch.manual_seed(42)``: the flash_attention.py teaching page,
``compare_and_verify``; the packed call of the flash-attn build guide,
section 5.2, draws one qkv tensor [B, N, 3, H, d]):

* a CPU ``torch.Generator`` seeded with ``seed`` (42 unless stated);
* Q, then K, then V, each ``randn`` of the full shape in float32;
* each cast to the requested dtype with round-to-nearest-even (``.to``).

Packed inputs draw one float32 tensor [B, N, 3, H, d] and split it.
"""

from __future__ import annotations

import hashlib

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

# The five workloads (shape, dtype, mask) the method is measured and checked on.
CONFIGS = {
    1: dict(name="single-head", B=1, H=1, N=256, D=64, dtype="f16", causal=False, packed=False),
    2: dict(name="packed-qkv", B=2, H=12, N=256, D=64, dtype="f16", causal=False, packed=True),
    3: dict(name="fp32-long", B=4, H=1, N=4096, D=64, dtype="f32", causal=False, packed=False),
    4: dict(name="gpt3-causal", B=1, H=128, N=2048, D=128, dtype="bf16", causal=True, packed=False),
    5: dict(name="long-causal-d256", B=1, H=16, N=16384, D=256, dtype="bf16", causal=True, packed=False),
}


def _dtype(dtype):
    if isinstance(dtype, torch.dtype):
        return dtype
    return DTYPES[dtype]


def make_qkv(B, H, N, D, dtype="bf16", seed=42):
    """Q, K, V as contiguous CPU tensors [B, H, N, D] of ``dtype``."""
    g = torch.Generator().manual_seed(seed)
    dt = _dtype(dtype)
    q = torch.randn(B, H, N, D, generator=g, dtype=torch.float32).to(dt)
    k = torch.randn(B, H, N, D, generator=g, dtype=torch.float32).to(dt)
    v = torch.randn(B, H, N, D, generator=g, dtype=torch.float32).to(dt)
    return q, k, v


def make_packed_qkv(B, N, H, D, dtype="f16", seed=42):
    """One packed tensor [B, N, 3, H, D] of ``dtype`` (the packed call's input)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, N, 3, H, D, generator=g, dtype=torch.float32).to(_dtype(dtype))


def unpack_qkv(qkv):
    """Split [B, N, 3, H, D] into three contiguous [B, H, N, D] tensors."""
    return tuple(qkv[:, :, i].permute(0, 2, 1, 3).contiguous() for i in range(3))


def make_config(cfg, seed=42):
    """Inputs (q, k, v) for one of the five workloads, in [B, H, N, D]."""
    c = CONFIGS[cfg]
    if c["packed"]:
        return unpack_qkv(make_packed_qkv(c["B"], c["N"], c["H"], c["D"], c["dtype"], seed))
    return make_qkv(c["B"], c["H"], c["N"], c["D"], c["dtype"], seed)


def make_cycled_heads(B, H, N, D, dtype, period, seed=42, device="cpu"):
    """Q, K, V [B, H, N, D] whose B*H heads repeat a pool of ``period``
    distinct seeded heads: flat head b*H + h is head (b*H + h) % period of
    ``make_qkv(1, period, N, D, dtype, seed)``. Builds tensors of many GB
    cheaply; the gather runs on ``device``."""
    idx = torch.arange(B * H, device=device) % period
    return tuple(p[0].to(device)[idx].view(B, H, N, D) for p in make_qkv(1, period, N, D, dtype, seed))


def digest(*tensors):
    """SHA-256 over the raw bytes of the given CPU tensors (input provenance)."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
