"""CPU model of the roundings of the 16-bit attention forward kernel.

Test infrastructure beside the fp64 oracle, not an oracle: the oracle
(``oracle/``) fixes what attention is and stays the parity bar; this model
fixes how the 16-bit kernel documents its arithmetic, so that a GPU test can
compare the kernel against a computation that rounds at the same places and
see kernel errors far below the rounding error of a bf16 output (which alone
reaches 7.8e-3 on rows whose |O| is near 2).

The arithmetic modelled (the online-softmax recurrence of
``flash_attention_forward`` on the flash_attention.py teaching page, in the
exp2 domain, with the kernel's lazy exponent reference):

* scores S = q . k in fp32 from the stored 16-bit inputs; c = fp32(scale *
  log2 e), with c = 0 replaced by the smallest normal float;
* query rows in blocks of ``Br`` (128), keys in tiles of ``Bc`` (64); a block
  visits the key tiles its rows can see (causal mask, window, fewer queries
  than keys: query row i at position i + Nk - N);
* per row, the exponent reference m starts at max(S) * c over the row's
  visible keys of the block's first tile (-inf if none); for every tile,
  P = exp2(fl32(S c - m)) (one rounding, as a fused multiply-add) and the
  fp32 row sum of P over the tile; if that sum is not <= 2^8 (P too large,
  or m still -inf) the row's m moves to max(m, tile max), the running sum
  and accumulator are scaled by exp2(m_old - m_new) and P is recomputed;
* l += the row sum of the unrounded P; acc += RNE_16(P) V in fp32;
* O = RNE_16(acc * fp32(1 / l)); LSE = (m + log2 l) ln 2.

With ``exact=True`` every step runs in float64 without the two 16-bit
roundings: the lazy reference then cancels exactly, so the result must equal
the plain definition to float64 rounding (a CPU test pins this).

Plain PyTorch CPU ops; shares nothing with the HIP library.
"""

from __future__ import annotations

import math

import numpy as np
import torch

_UNBOUNDED = 1 << 30
_FLT_MIN = 1.17549435e-38


def _round16(x32, dtype):
    """Round-to-nearest-even of fp32 values to the 16-bit input type, back in fp32."""
    return x32.to(dtype).to(torch.float32)


def forward_model(q, k, v, scale, causal=False, window=(-1, -1), Br=128, Bc=64, exact=False):
    """(O, LSE) of the modelled kernel for CPU tensors q [B, H, N, d] and k, v
    [B, H, Nk, d] of one 16-bit dtype. O comes back in that dtype (exact:
    float64), LSE in float32 (exact: float64)."""
    dtype = q.dtype
    if not exact and dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("the rounding model covers the 16-bit kernel (fp16 / bf16 inputs)")
    B, H, N, D = q.shape
    Nk = k.shape[2]
    ft = torch.float64 if exact else torch.float32
    qf = q.reshape(B * H, N, D).to(ft)
    kf = k.reshape(B * H, Nk, D).to(ft)
    vf = v.reshape(B * H, Nk, D).to(ft)
    # The kernel flips the sign of q for a negative scale and uses |c| (the
    # same products), and replaces c = 0 by the smallest normal float.
    cval = abs(scale * 1.4426950408889634074) if exact else abs(float(np.float32(scale * 1.4426950408889634074)))
    c = torch.tensor(cval if cval != 0.0 else _FLT_MIN, dtype=ft)
    if scale < 0:
        qf = -qf
    wl = _UNBOUNDED if window[0] < 0 else int(window[0])
    wr = _UNBOUNDED if window[1] < 0 else int(window[1])
    if causal:
        wr = 0
    pos_off = Nk - N
    out = torch.empty(B * H, N, D, dtype=ft)
    lse = torch.empty(B * H, N, dtype=ft)
    tau = torch.tensor(256.0, dtype=ft)
    for r0 in range(0, N, Br):
        r1 = min(r0 + Br, N)
        pos = torch.arange(r0, r1) + pos_off
        p_lo = r0 + pos_off
        t_lo = max(p_lo - wl, 0) // Bc
        t_hi = min(min(r0 + Br - 1, N - 1) + pos_off + wr, Nk - 1) // Bc
        qb = qf[:, r0:r1]
        m = torch.full((B * H, r1 - r0), -math.inf, dtype=ft)
        l = torch.zeros(B * H, r1 - r0, dtype=ft)
        acc = torch.zeros(B * H, r1 - r0, D, dtype=ft)
        for t in range(t_lo, t_hi + 1):
            k0, k1 = t * Bc, min(t * Bc + Bc, Nk)
            keys = torch.arange(k0, k1)
            vis = (keys[None, :] <= pos[:, None] + wr) & (keys[None, :] >= pos[:, None] - wl)
            s = torch.bmm(qb, kf[:, k0:k1].transpose(1, 2))
            s = torch.where(vis[None], s, torch.tensor(-math.inf, dtype=ft))
            smax = s.max(dim=2).values
            tmax = torch.where(torch.isneginf(smax), smax, smax * c)
            if t == t_lo:
                m = tmax

            def expo(ref):
                # exp2(fl32(S c - ref)): the product is exact in float64 and the
                # difference is rounded once to fp32, as a fused multiply-add.
                if exact:
                    return torch.exp2(s * c - ref[..., None])
                arg = (s.double() * c.double() - ref.double()[..., None]).float()
                return torch.exp2(arg)

            p = expo(m)
            ls = p.sum(dim=2)
            need = ~(ls <= tau)
            if bool(need.any()):
                m_new = torch.where(need, torch.maximum(m, tmax), m)
                m_use = torch.where(torch.isneginf(m_new), torch.zeros_like(m_new), m_new)
                alpha = torch.exp2(m - m_use)
                m = m_new
                p = expo(m_use)
                ls = p.sum(dim=2)
                l = l * alpha
                acc = acc * alpha[..., None]
            l = l + ls
            pv = p if exact else _round16(p, dtype)
            acc = acc + torch.bmm(pv, vf[:, k0:k1])
        if exact:
            out[:, r0:r1] = acc / l[..., None]
            lse[:, r0:r1] = (m + torch.log2(l)) * math.log(2.0)
        else:
            inv = (1.0 / l).float()
            out[:, r0:r1] = acc * inv[..., None]
            lse[:, r0:r1] = (m + torch.log2(l)) * np.float32(math.log(2.0))
    o = out.view(B, H, N, D)
    return (o if exact else o.to(dtype)), lse.view(B, H, N)


def output_ulp(o, dtype):
    """Spacing of the 16-bit output type at |o| (float64 array): 2^(e - p + 1)
    for |o| in [2^e, 2^(e+1)), with p = 8 (bf16) or 11 (fp16); subnormal and
    zero magnitudes get the spacing at the smallest normal."""
    p = 8 if dtype == torch.bfloat16 else 11
    emin = -126 if dtype == torch.bfloat16 else -14
    a = np.abs(np.asarray(o, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, emin), emin)
    return np.exp2(e - p + 1)
