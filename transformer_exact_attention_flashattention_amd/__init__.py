"""Exact-attention forward pass on MI355X (gfx950): thin Python binding.

Every step of the computation runs in the HIP kernels of ``libfa.so``; this
module only marshals arguments (device pointers, sizes, the current stream)
into the C ABI declared in ``include/fa.h``. There is no CPU fallback: if the
library is missing or the tensors are not on a GPU, the calls raise.

API (names follow the flash-attn interface that section 5.2 / 10.1 of the
flash-attn 2.8.3 build guide, intelliparadigm.com, calls):

* ``fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1))
  -> (o, lse)`` with q, k, v of shape [B, H, N, d] (the layout of section 1.1
  of "2.3 FlashAttention and IO-aware attention") on one GPU, all of dtype
  float16, bfloat16 or float32. Any strides are accepted as long as the last
  dimension is contiguous and rows are 16-byte aligned (a transposed view of
  a [B, N, H, d] tensor is read in place); ``softmax_scale=None`` means
  1/sqrt(d); ``window_size=(left, right)`` restricts query i to keys
  i - left .. i + right (-1: unbounded side), the reading of the
  ``window_size`` argument that section 10.1 lists.
* ``flash_attn_qkvpacked_func(qkv, dropout_p=0.0, softmax_scale=None,
  causal=False, window_size=(-1, -1)) -> o`` for a packed tensor
  [B, N, 3, H, d] (section 5.2): o is [B, N, H, d]. The q, k and v slices are
  read in place (no copy), and the call is differentiable: its backward
  writes the gradient of the packed tensor in place too.
* ``flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None,
  causal=False, window_size=(-1, -1)) -> o`` for q, k, v of shape
  [B, N, H, d] (the per-tensor form of the packed layout), o [B, N, H, d];
  differentiable.
* ``bwd(q, k, v, o, lse, do, softmax_scale=None, causal=False,
  window_size=(-1, -1)) -> (dq, dk, dv)``: the backward pass (fp16/bf16,
  d = 64, 128 or 256), recomputing the attention weights from q, k and the
  forward's lse (section 9.2 item 2 of the build guide); strided views as
  for ``fwd``, including the gradients passed in as dq, dk, dv.
* ``attention(q, k, v, softmax_scale=None, causal=False,
  window_size=(-1, -1)) -> o``: [B, H, N, d], differentiable through torch
  autograd; its backward calls ``bwd``.
* ``fa_fwd(...)``, ``fa_fwd_window(...)``, ``fa_fwd_strided(...)``,
  ``fa_bwd(...)``, ``fa_bwd_strided(...)``: the raw C entry points with the
  same arguments as the C functions (strides as a sequence of ints or None),
  for callers that manage their own pointers and streams;
  ``fa_fwd_strided_check(...)`` and ``fa_bwd_strided_check(...)`` run only
  their host-side argument checks.
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
    -8: "FA_ERR_SCRATCH",
}
# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_window", "fa_fwd_strided", "fa_bwd", "fa_bwd_strided", "fa_strerror",
           "fa_fwd_grid", "fa_fwd_strided_check", "fa_bwd_strided_check", "fa_fwd_splitkv",
           "fa_fwd_num_splits", "fa_fwd_splitkv_workspace", "fa_fwd_kv", "fa_fwd_kv_num_splits",
           "fa_fwd_kv_noalloc")
# Bytes of the static device array behind fa_fwd_kv_noalloc (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20

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
        h.fa_fwd_strided.restype = ctypes.c_int
        h.fa_fwd_strided.argtypes = [ctypes.c_void_p] * 5 + [ctypes.POINTER(ctypes.c_longlong)] + [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_bwd.restype = ctypes.c_int
        h.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_bwd_strided.restype = ctypes.c_int
        h.fa_bwd_strided.argtypes = [ctypes.c_void_p] * 10 + [ctypes.POINTER(ctypes.c_longlong)] + [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_fwd_splitkv.restype = ctypes.c_int
        h.fa_fwd_splitkv.argtypes = [ctypes.c_void_p] * 5 + [
            ctypes.POINTER(ctypes.c_longlong), ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_fwd_kv.restype = ctypes.c_int
        h.fa_fwd_kv.argtypes = [ctypes.c_void_p] * 5 + [
            ctypes.POINTER(ctypes.c_longlong), ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_fwd_kv_noalloc.restype = ctypes.c_int
        h.fa_fwd_kv_noalloc.argtypes = [ctypes.c_void_p] * 5 + [
            ctypes.POINTER(ctypes.c_longlong), ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        h.fa_fwd_kv_num_splits.restype = ctypes.c_int
        h.fa_fwd_kv_num_splits.argtypes = [ctypes.c_int] * 9 + [ctypes.POINTER(ctypes.c_int)]
        h.fa_fwd_num_splits.restype = ctypes.c_int
        h.fa_fwd_num_splits.argtypes = [ctypes.c_int] * 8 + [ctypes.POINTER(ctypes.c_int)]
        h.fa_fwd_splitkv_workspace.restype = ctypes.c_int
        h.fa_fwd_splitkv_workspace.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_longlong)]
        h.fa_fwd_strided_check.restype = ctypes.c_int
        h.fa_fwd_strided_check.argtypes = h.fa_fwd_strided.argtypes[:-1]
        h.fa_bwd_strided_check.restype = ctypes.c_int
        h.fa_bwd_strided_check.argtypes = h.fa_bwd_strided.argtypes[:-1]
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


def _strides_arg(strides, n):
    if strides is None:
        return None
    vals = [int(x) for x in strides]
    if len(vals) != n:
        raise ValueError(f"expected {n} strides, got {len(vals)}")
    return (ctypes.c_longlong * n)(*vals)


def fa_fwd_strided(q, k, v, o, lse, strides, B, H, N, d, scale, causal, window_left, window_right, dtype,
                   stream=None) -> int:
    """Raw call of the strided C entry point: strides holds 12 element
    strides (batch, head, row of q, k, v, o) or is None (contiguous)."""
    return lib().fa_fwd_strided(q, k, v, o, lse, _strides_arg(strides, 12), B, H, N, d, scale, causal,
                                window_left, window_right, dtype, stream)


def fa_fwd_splitkv(q, k, v, o, lse, strides, workspace, workspace_bytes, num_splits, B, H, N, d, scale, causal,
                   window_left, window_right, dtype, stream=None) -> int:
    """Raw call of the split-KV entry point (strides as for fa_fwd_strided)."""
    return lib().fa_fwd_splitkv(q, k, v, o, lse, _strides_arg(strides, 12), workspace, workspace_bytes, num_splits,
                                B, H, N, d, scale, causal, window_left, window_right, dtype, stream)


def fa_fwd_kv(q, k, v, o, lse, strides, workspace, workspace_bytes, num_splits, B, H, N, Nk, d, scale, causal,
              window_left, window_right, dtype, stream=None) -> int:
    """Raw call of the general forward: N query rows against Nk key rows."""
    return lib().fa_fwd_kv(q, k, v, o, lse, _strides_arg(strides, 12), workspace, workspace_bytes, num_splits,
                           B, H, N, Nk, d, scale, causal, window_left, window_right, dtype, stream)


def fa_fwd_kv_noalloc(q, k, v, o, lse, strides, num_splits, B, H, N, Nk, d, scale, causal, window_left,
                      window_right, dtype, stream=None) -> int:
    """Raw call of the allocation-free general forward (split-KV partial
    results in the library's static device array; no workspace)."""
    return lib().fa_fwd_kv_noalloc(q, k, v, o, lse, _strides_arg(strides, 12), num_splits, B, H, N, Nk, d, scale,
                                   causal, window_left, window_right, dtype, stream)


def splitkv_num_splits(B, H, N, d, causal=False, window_size=(-1, -1), dtype=FA_BF16, Nk=None):
    """The number of key-range parts the split-KV forward picks by itself
    (for N queries against Nk keys; Nk defaults to N)."""
    left, right = _window(window_size)
    n = ctypes.c_int(0)
    nk = N if Nk is None else int(Nk)
    st = lib().fa_fwd_kv_num_splits(B, H, N, nk, d, int(bool(causal)), left, right, dtype, ctypes.byref(n))
    if st != 0:
        raise FaError(st, strerror(st))
    return n.value


def splitkv_workspace_bytes(B, H, N, d, splits):
    """Workspace bytes fa_fwd_splitkv needs for ``splits`` parts."""
    n = ctypes.c_longlong(0)
    st = lib().fa_fwd_splitkv_workspace(B, H, N, d, splits, ctypes.byref(n))
    if st != 0:
        raise FaError(st, strerror(st))
    return n.value


def fa_fwd_strided_check(q, k, v, o, lse, strides, B, H, N, d, scale, causal, window_left, window_right,
                         dtype) -> int:
    """Status fa_fwd_strided would return from its checks; no HIP call."""
    return lib().fa_fwd_strided_check(q, k, v, o, lse, _strides_arg(strides, 12), B, H, N, d, scale, causal,
                                      window_left, window_right, dtype)


def fa_bwd_strided_check(q, k, v, o, lse, do, dq, dk, dv, delta, strides, B, H, N, d, scale, causal,
                         window_left, window_right, dtype) -> int:
    """Status fa_bwd_strided would return from its checks; no HIP call."""
    return lib().fa_bwd_strided_check(q, k, v, o, lse, do, dq, dk, dv, delta, _strides_arg(strides, 24), B, H,
                                      N, d, scale, causal, window_left, window_right, dtype)


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, N, d, scale, causal, window_left,
           window_right, dtype, stream=None) -> int:
    """Raw call of the backward C entry point; pointers are ints (device addresses)."""
    return lib().fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, N, d, scale, causal, window_left,
                        window_right, dtype, stream)


def fa_bwd_strided(q, k, v, o, lse, do, dq, dk, dv, delta, strides, B, H, N, d, scale, causal, window_left,
                   window_right, dtype, stream=None) -> int:
    """Raw call of the strided backward entry point: strides holds 24 element
    strides (batch, head, row of q, k, v, o, do, dq, dk, dv) or is None."""
    return lib().fa_bwd_strided(q, k, v, o, lse, do, dq, dk, dv, delta, _strides_arg(strides, 24), B, H, N, d,
                                scale, causal, window_left, window_right, dtype, stream)


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


def _check_view(name, t, shape, dtype, device):
    """A [B, H, N, d] operand: a GPU tensor of the given shape, dtype and
    device whose last dimension is contiguous; other strides are checked by
    the library."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")


def _check_rowstat(name, t, B, H, N, device):
    import torch

    if t.shape != (B, H, N) or t.dtype != torch.float32 or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 tensor [B, H, N] on q's device")


def _strides(*ts):
    out = []
    for t in ts:
        out.extend(t.stride()[:3])
    return out


def fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), out=None, lse=None, num_splits=1,
        workspace=None):
    """Attention forward on the GPU: returns (o [B,H,N,d], lse [B,H,N] fp32).

    q, k, v (and ``out`` if given) may be strided views; a new ``out`` is
    contiguous. k and v may have more rows than q ([B, H, Nk, d], a key/value
    cache): the queries are then the last N positions (fa_fwd_kv).
    ``num_splits`` > 1 splits every query tile's keys into that many parts
    merged by log-sum-exp; 0 lets the library choose; the workspace (a GPU
    tensor of at least ``splitkv_workspace_bytes`` bytes) is allocated when
    not given."""
    import torch

    left, right = _window(window_size)
    _check_view("q", q, None, None, None)
    code = _dtype_code(q)
    _check_view("k", k, None, q.dtype, q.device)
    kv_shape = (q.shape[0], q.shape[1], k.shape[2], q.shape[3])
    if tuple(k.shape) != kv_shape:
        raise ValueError(f"k must be [B, H, Nk, d] with q's B, H, d: q {tuple(q.shape)}, k {tuple(k.shape)}")
    _check_view("v", v, kv_shape, q.dtype, q.device)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if d not in (64, 128, 256):
        raise NotImplementedError(f"head dimension {d} is not supported (64, 128, 256)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_view("out", out, q.shape, q.dtype, q.device)
    _check_rowstat("lse", lse, B, H, N, q.device)
    splits = int(num_splits)
    if splits == 0:
        splits = splitkv_num_splits(B, H, N, d, causal, (left, right), code, Nk=Nk)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        if splits == 1 and Nk == N:
            st = fa_fwd_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), _strides(q, k, v, out),
                B, H, N, d, scale, int(bool(causal)), left, right, code, stream,
            )
        else:
            need = splitkv_workspace_bytes(B, H, N, d, splits)
            if workspace is None and need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            if workspace is not None and (not workspace.is_cuda or workspace.device != q.device):
                raise ValueError("workspace must be on q's device")
            ws_ptr = workspace.data_ptr() if workspace is not None else None
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            st = fa_fwd_kv(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), _strides(q, k, v, out),
                ws_ptr, ws_bytes, splits, B, H, N, Nk, d, scale, int(bool(causal)), left, right, code, stream,
            )
    if st != 0:
        raise FaError(st, strerror(st))
    return out, lse


def bwd(q, k, v, o, lse, do, softmax_scale=None, causal=False, window_size=(-1, -1), dq=None, dk=None,
        dv=None, delta=None):
    """Backward pass on the GPU: returns (dq, dk, dv), each of q's shape.

    o and lse are the forward's outputs for the same q, k, v, scale, causal
    and window; do is the gradient of the loss with respect to o. Every
    [B, H, N, d] operand may be a strided view (new gradients are
    contiguous). ``delta`` (optional, [B, H, N] float32) receives
    rowsum(do * o)."""
    import torch

    left, right = _window(window_size)
    _check_view("q", q, None, None, None)
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check_view(name, t, q.shape, q.dtype, q.device)
    code = _dtype_code(q)
    if code == FA_F32:
        raise NotImplementedError("the backward pass supports float16 and bfloat16")
    B, H, N, d = q.shape
    if d not in (64, 128, 256):
        raise NotImplementedError(f"head dimension {d} is not supported (64, 128, 256)")
    _check_rowstat("lse", lse, B, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    new = lambda: torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)  # noqa: E731
    dq = new() if dq is None else dq
    dk = new() if dk is None else dk
    dv = new() if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_view(name, t, q.shape, q.dtype, q.device)
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_rowstat("delta", delta, B, H, N, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = fa_bwd_strided(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), _strides(q, k, v, o, do, dq, dk, dv),
            B, H, N, d, scale, int(bool(causal)), left, right, code, stream,
        )
    if st != 0:
        raise FaError(st, strerror(st))
    return dq, dk, dv


def _last_dim_contiguous(t):
    return t if t.shape[-1] <= 1 or t.stride(-1) == 1 else t.contiguous()


_autograd_fns = None


def _autograd_functions():
    """The torch.autograd.Function classes (built on first use, so that the
    module imports without torch)."""
    global _autograd_fns
    if _autograd_fns is None:
        import torch

        class _Attention(torch.autograd.Function):
            """q, k, v [B, H, N, d] (or [B, N, H, d] with bnhd=True) -> o of
            the same layout."""

            @staticmethod
            def forward(ctx, q, k, v, softmax_scale, causal, window_size, bnhd):
                t = (lambda x: x.transpose(1, 2)) if bnhd else (lambda x: x)
                o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
                _, lse = fwd(t(q), t(k), t(v), softmax_scale=softmax_scale, causal=causal,
                             window_size=window_size, out=t(o))
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.args = (softmax_scale, causal, window_size, bnhd)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                softmax_scale, causal, window_size, bnhd = ctx.args
                if k.shape != q.shape:
                    raise NotImplementedError("the backward pass needs equal query and key lengths")
                t = (lambda x: x.transpose(1, 2)) if bnhd else (lambda x: x)
                grads = [torch.empty(q.shape, dtype=q.dtype, device=q.device) for _ in range(3)]
                bwd(t(q), t(k), t(v), t(o), lse, t(_last_dim_contiguous(do)), softmax_scale=softmax_scale,
                    causal=causal, window_size=window_size, dq=t(grads[0]), dk=t(grads[1]), dv=t(grads[2]))
                return grads[0], grads[1], grads[2], None, None, None, None

        class _AttentionQKVPacked(torch.autograd.Function):
            """qkv [B, N, 3, H, d] -> o [B, N, H, d]; q, k, v and their
            gradients are slices of the packed tensors, used in place."""

            @staticmethod
            def forward(ctx, qkv, softmax_scale, causal, window_size):
                B, N, _, H, d = qkv.shape
                o = torch.empty((B, N, H, d), dtype=qkv.dtype, device=qkv.device)
                sl = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
                _, lse = fwd(*sl, softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                             out=o.transpose(1, 2))
                ctx.save_for_backward(qkv, o, lse)
                ctx.args = (softmax_scale, causal, window_size)
                return o

            @staticmethod
            def backward(ctx, do):
                qkv, o, lse = ctx.saved_tensors
                softmax_scale, causal, window_size = ctx.args
                dqkv = torch.empty(qkv.shape, dtype=qkv.dtype, device=qkv.device)
                sl = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
                gl = [dqkv[:, :, i].transpose(1, 2) for i in range(3)]
                bwd(*sl, o.transpose(1, 2), lse, _last_dim_contiguous(do).transpose(1, 2),
                    softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                    dq=gl[0], dk=gl[1], dv=gl[2])
                return dqkv, None, None, None

        _autograd_fns = (_Attention, _AttentionQKVPacked)
    return _autograd_fns


def attention(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1)):
    """Differentiable attention: o = softmax(scale q k^T [+ masks]) v for
    q, k, v [B, H, N, d], with ``fwd`` forward and ``bwd`` backward under
    torch autograd."""
    return _autograd_functions()[0].apply(q, k, v, softmax_scale, causal, tuple(_window(window_size)), False)


def _no_dropout(dropout_p, alibi_slopes=None):
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    if alibi_slopes is not None:
        raise NotImplementedError("ALiBi is not supported")


def flash_attn_qkvpacked_func(qkv, dropout_p=0.0, softmax_scale=None, causal=False,
                              window_size=(-1, -1), alibi_slopes=None, deterministic=False):
    """Packed-QKV attention: qkv [B, N, 3, H, d] -> o [B, N, H, d],
    differentiable. The slices of qkv are read in place; the backward is
    deterministic whatever ``deterministic`` says (no atomics)."""
    _no_dropout(dropout_p, alibi_slopes)
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError(f"qkv must be [B, N, 3, H, d], got {tuple(qkv.shape)}")
    return _autograd_functions()[1].apply(qkv, softmax_scale, causal, tuple(_window(window_size)))


def flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                    alibi_slopes=None, deterministic=False):
    """Attention for q [B, N, H, d] and k, v [B, Nk, H, d] -> o [B, N, H, d],
    differentiable when Nk = N; inputs are read in place (any strides with a
    contiguous last dimension). With Nk > N the queries are the last N
    positions (a key/value cache)."""
    _no_dropout(dropout_p, alibi_slopes)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, N, H, d], got shape {tuple(t.shape)}")
    return _autograd_functions()[0].apply(q, k, v, softmax_scale, causal, tuple(_window(window_size)), True)
