"""Exact-attention forward pass on MI355X (gfx950): thin Python binding.

Every step of the computation runs in the HIP kernels of ``libfa.so``; this
module only marshals arguments (device pointers, sizes, the current stream)
into the C ABI declared in ``include/fa.h``. There is no CPU fallback: if the
library is missing or the tensors are not on a GPU, the calls raise.

API (names follow the flash-attn interface that section 5.2 / 10.1 of the
flash-attn 2.8.3 build guide, intelliparadigm.com, calls):

* ``fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1))
  -> (o, lse)`` with q, k, v of shape [B, H, N, d] (the layout of section 1.1
  of "2.3 FlashAttention and IO-aware attention"), contiguous, on one GPU,
  all of dtype float16, bfloat16 or float32; ``softmax_scale=None`` means
  1/sqrt(d); ``window_size=(left, right)`` restricts query i to keys
  i - left .. i + right (-1: unbounded side), the reading of the
  ``window_size`` argument that section 10.1 lists.
* ``flash_attn_qkvpacked_func(qkv, dropout_p=0.0, softmax_scale=None,
  causal=False) -> (o, lse)`` for a packed tensor [B, N, 3, H, d]; it splits
  and transposes the packed tensor into three [B, H, N, d] tensors (a copy)
  and calls ``fwd``; o and lse come back as [B, H, N, d] and [B, H, N].
* ``bwd(q, k, v, o, lse, do, softmax_scale=None, causal=False,
  window_size=(-1, -1)) -> (dq, dk, dv)``: the backward pass (fp16/bf16,
  d = 64 or 128), recomputing the attention weights from q, k and the
  forward's lse (section 9.2 item 2 of the build guide).
* ``attention(q, k, v, softmax_scale=None, causal=False,
  window_size=(-1, -1)) -> o``: differentiable through torch autograd; its
  backward calls ``bwd``.
* ``fa_fwd(...)``, ``fa_fwd_window(...)``, ``fa_bwd(...)``: the raw C entry
  points with the same arguments as the C functions, for callers that manage
  their own pointers and streams.
"""

from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

FA_F16, FA_BF16, FA_F32 = 0, 1, 2
STATUS = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_SHAPE",
    -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_ALIGN",
    -6: "FA_ERR_ARG",
    -7: "FA_ERR_LAUNCH",
}
# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_window", "fa_bwd", "fa_strerror", "fa_fwd_grid")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run "
                "`python -c 'import __graft_entry__ as g; g.build()'` first"
            )
        h = ctypes.CDLL(LIB_PATH)
        h.fa_fwd.restype = ctypes.c_int
        h.fa_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_fwd_window.restype = ctypes.c_int
        h.fa_fwd_window.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_bwd.restype = ctypes.c_int
        h.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_strerror.restype = ctypes.c_char_p
        h.fa_strerror.argtypes = [ctypes.c_int]
        h.fa_fwd_grid.restype = ctypes.c_int
        h.fa_fwd_grid.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_int),
        ]
        _lib = h
    return _lib


def strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream=None) -> int:
    """Raw call of the C entry point; pointers are ints (device addresses)."""
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream)


def fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, causal, window_left, window_right, dtype,
                  stream=None) -> int:
    """Raw call of the windowed C entry point; pointers are ints (device addresses)."""
    return lib().fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, causal, window_left, window_right,
                               dtype, stream)


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, N, d, scale, causal, window_left,
           window_right, dtype, stream=None) -> int:
    """Raw call of the backward C entry point; pointers are ints (device addresses)."""
    return lib().fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, N, d, scale, causal, window_left,
                        window_right, dtype, stream)


def _window(window_size):
    try:
        left, right = (int(w) for w in window_size)
    except (TypeError, ValueError):
        raise ValueError(f"window_size must be a pair of ints, got {window_size!r}") from None
    if left < -1 or right < -1:
        raise ValueError(f"window_size sides must be >= -1 (-1: unbounded), got {window_size!r}")
    return left, right


def grid(B, H, N, d, causal, dtype):
    """(workgroups, query rows per workgroup) of the launch fa_fwd would make."""
    wg = ctypes.c_longlong(0)
    rows = ctypes.c_int(0)
    st = lib().fa_fwd_grid(B, H, N, d, int(causal), dtype, ctypes.byref(wg), ctypes.byref(rows))
    if st != 0:
        raise FaError(st, strerror(st))
    return wg.value, rows.value


def _dtype_code(t):
    import torch

    codes = {torch.float16: FA_F16, torch.bfloat16: FA_BF16, torch.float32: FA_F32}
    if t.dtype not in codes:
        raise NotImplementedError(f"dtype {t.dtype} is not supported (float16, bfloat16, float32)")
    return codes[t.dtype]


def fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), out=None, lse=None):
    """Attention forward on the GPU: returns (o [B,H,N,d], lse [B,H,N] fp32)."""
    import torch

    left, right = _window(window_size)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    code = _dtype_code(q)
    B, H, N, d = q.shape
    if d not in (64, 128, 256):
        raise NotImplementedError(f"head dimension {d} is not supported (64, 128, 256)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib().fa_fwd_window(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, N, d, scale, int(bool(causal)), left, right, code, stream,
        )
    if st != 0:
        raise FaError(st, strerror(st))
    return out, lse


def flash_attn_qkvpacked_func(qkv, dropout_p=0.0, softmax_scale=None, causal=False,
                              window_size=(-1, -1), alibi_slopes=None, deterministic=False):
    """Packed-QKV entry: qkv [B, N, 3, H, d] -> (o [B,H,N,d], lse [B,H,N])."""
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    if alibi_slopes is not None:
        raise NotImplementedError("ALiBi is not supported")
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError(f"qkv must be [B, N, 3, H, d], got {tuple(qkv.shape)}")
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3).contiguous() for i in range(3))
    return fwd(q, k, v, softmax_scale=softmax_scale, causal=causal, window_size=window_size)


def flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1)):
    """Same as ``fwd`` (q, k, v in [B, H, N, d]); dropout must be 0."""
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    return fwd(q, k, v, softmax_scale=softmax_scale, causal=causal, window_size=window_size)


def bwd(q, k, v, o, lse, do, softmax_scale=None, causal=False, window_size=(-1, -1), dq=None, dk=None,
        dv=None, delta=None):
    """Backward pass on the GPU: returns (dq, dk, dv), each like q.

    o and lse are the forward's outputs for the same q, k, v, scale, causal
    and window; do is the gradient of the loss with respect to o. ``delta``
    (optional, [B, H, N] float32) receives rowsum(do * o)."""
    import torch

    left, right = _window(window_size)
    ts = (("q", q), ("k", k), ("v", v), ("o", o), ("do", do))
    for name, t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
        if t.shape != q.shape or t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d] like q, got {tuple(t.shape)}")
        if t.dtype != q.dtype or t.device != q.device:
            raise TypeError(f"{name} must match q's dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    code = _dtype_code(q)
    if code == FA_F32:
        raise NotImplementedError("the backward pass supports float16 and bfloat16")
    B, H, N, d = q.shape
    if d not in (64, 128):
        raise NotImplementedError(f"head dimension {d} is not supported by the backward pass (64, 128)")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if delta.shape != (B, H, N) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 tensor [B, H, N]")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib().fa_bwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
            B, H, N, d, scale, int(bool(causal)), left, right, code, stream,
        )
    if st != 0:
        raise FaError(st, strerror(st))
    return dq, dk, dv


_autograd_fn = None


def _attention_function():
    global _autograd_fn
    if _autograd_fn is None:
        import torch

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, softmax_scale, causal, window_size):
                o, lse = fwd(q, k, v, softmax_scale=softmax_scale, causal=causal, window_size=window_size)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.args = (softmax_scale, causal, window_size)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                softmax_scale, causal, window_size = ctx.args
                dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), softmax_scale=softmax_scale, causal=causal,
                                 window_size=window_size)
                return dq, dk, dv, None, None, None

        _autograd_fn = _Attention
    return _autograd_fn


def attention(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1)):
    """Differentiable attention: o = softmax(scale q k^T [+ masks]) v, with
    ``fwd`` forward and ``bwd`` backward under torch autograd."""
    return _attention_function().apply(q, k, v, softmax_scale, causal, tuple(window_size))
