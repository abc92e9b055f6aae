"""Fused, chunked top-K KL distillation loss on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libkdkl.so`` (C ABI in ``include/kdkl.h``).  Every
step of the computation runs in the library's HIP kernels; this module only
allocates outputs and the workspace with torch and passes pointers and the
current HIP stream.  There is no fallback: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["KDError", "library_path", "workspace_bytes", "fwd_bwd", "fwd", "bwd",
           "chunked_kl_loss", "scale_grads", "teacher_topk", "vocab_shard_fwd", "vocab_shard_combine",
           "vocab_shard_bwd", "profile_enable", "profile_read", "profile_classes", "KD_F32",
           "KD_BF16"]

KD_F32, KD_BF16 = 0, 1
_STATUS = {0: "KD_OK", 1: "KD_E_ARG", 2: "KD_E_INDEX", 3: "KD_E_WORKSPACE",
           4: "KD_E_UNSUPPORTED", 5: "KD_E_HIP"}

_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdkl.so")


class KDError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.kd_workspace_bytes.argtypes = [i64, i64, i64, i32, i64, i32, ctypes.POINTER(sz)]
    lib.kd_workspace_bytes.restype = ctypes.c_int
    lib.kd_workspace_bytes_group.argtypes = [i64, i64, i64, i32, i64, i32, i64,
                                             ctypes.POINTER(sz)]
    lib.kd_workspace_bytes_group.restype = ctypes.c_int
    lib.kd_chunked_kl_fwd_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, i64,
                                          vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd_bwd.restype = ctypes.c_int
    lib.kd_chunked_kl_fwd_bwd_async.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, i64,
                                                vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd_bwd_async.restype = ctypes.c_int
    lib.kd_chunked_kl_fwd_bwd_f32dh.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32,
                                                i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd_bwd_f32dh.restype = ctypes.c_int
    lib.kd_scale_grads.argtypes = [vp, vp, vp, i32, i64, i64, vp, i64, vp]
    lib.kd_scale_grads.restype = ctypes.c_int
    lib.kd_chunked_kl_fwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, i64,
                                      vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd.restype = ctypes.c_int
    lib.kd_chunked_kl_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, i64,
                                      vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_bwd.restype = ctypes.c_int
    lib.kd_vocab_shard_fwd.argtypes = [vp, vp, i32, vp, vp, i64, i64, i64, i64, i64, i32, i64,
                                       vp, vp, vp, vp, vp, sz, vp]
    lib.kd_vocab_shard_fwd.restype = ctypes.c_int
    lib.kd_vocab_shard_combine_workspace_bytes.argtypes = [i64, ctypes.POINTER(sz)]
    lib.kd_vocab_shard_combine_workspace_bytes.restype = ctypes.c_int
    lib.kd_vocab_shard_combine.argtypes = [vp, vp, vp, i32, vp, vp, i64, i32, vp, vp, vp, vp, sz,
                                           vp]
    lib.kd_vocab_shard_combine.restype = ctypes.c_int
    lib.kd_vocab_shard_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                       i64, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_vocab_shard_bwd.restype = ctypes.c_int
    lib.kd_topk_workspace_bytes.argtypes = [ctypes.POINTER(sz)]
    lib.kd_topk_workspace_bytes.restype = ctypes.c_int
    lib.kd_teacher_topk.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, sz, vp]
    lib.kd_teacher_topk.restype = ctypes.c_int
    lib.kd_teacher_topk_noalloc.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp]
    lib.kd_teacher_topk_noalloc.restype = ctypes.c_int
    lib.kd_last_error.argtypes = []
    lib.kd_last_error.restype = ctypes.c_char_p
    lib.kd_version.restype = ctypes.c_int
    lib.kd_profile_enable.argtypes = [ctypes.c_int]
    lib.kd_profile_num_classes.restype = ctypes.c_int
    lib.kd_profile_class_name.argtypes = [ctypes.c_int]
    lib.kd_profile_class_name.restype = ctypes.c_char_p
    lib.kd_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.kd_clock_stamp.argtypes = [vp, i32, vp]
    lib.kd_clock_stamp.restype = ctypes.c_int
    lib.kd_wall_clock_khz.argtypes = [ctypes.POINTER(i32)]
    lib.kd_wall_clock_khz.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise KDError(rc, _lib().kd_last_error().decode())


def workspace_bytes(N: int, d: int, V: int, K: int, chunk: int, dtype: int = KD_BF16,
                    dw_group_tokens: Optional[int] = None) -> int:
    """Workspace bytes: for the default dW group (``dw_group_tokens=None``) or for groups
    of at most ``dw_group_tokens`` tokens (0 = one chunk, the smallest accepted)."""
    out = ctypes.c_size_t(0)
    if dw_group_tokens is None:
        _check(_lib().kd_workspace_bytes(N, d, V, K, chunk, dtype, ctypes.byref(out)))
    else:
        _check(_lib().kd_workspace_bytes_group(N, d, V, K, chunk, dtype, dw_group_tokens,
                                               ctypes.byref(out)))
    return int(out.value)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KD_BF16
    if t.dtype == torch.float32:
        return KD_F32
    raise TypeError(f"h and W must be bfloat16 or float32, not {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_device(dev, **tensors):
    """Every tensor argument must live on ``dev``, a CUDA device: the library receives
    bare addresses and would read a host or another GPU's address as its own."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be CUDA tensors, got device {dev}")
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} is on {t.device}; every tensor argument must be on {dev}")


def _prep(h, W, topk_idx, topk_p, loss_mask):
    """Checks dtypes, shapes and contiguity; returns (dtype code, N, d, V, K, mask)."""
    import torch
    dt = _dtype_code(h)
    if W.dtype != h.dtype:
        raise TypeError("h and W must have the same dtype")
    if topk_idx.dtype != torch.int32 or topk_p.dtype != torch.float32:
        raise TypeError("topk_idx must be int32 and topk_p float32")
    _on_device(h.device, h=h, W=W, topk_idx=topk_idx, topk_p=topk_p, loss_mask=loss_mask)
    tensors = [h, W, topk_idx, topk_p] + ([loss_mask] if loss_mask is not None else [])
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    N, d = h.shape
    V, d2 = W.shape
    K = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if d2 != d or tuple(topk_idx.shape) != (N, K) or tuple(topk_p.shape) != (N, K):
        raise ValueError("shape mismatch among h, W, topk_idx and topk_p")
    if loss_mask is not None:
        if loss_mask.dtype == torch.bool:
            loss_mask = loss_mask.view(torch.uint8)
        if loss_mask.dtype != torch.uint8 or tuple(loss_mask.shape) != (N,):
            raise ValueError("loss_mask must be uint8/bool of shape [N]")
    return dt, N, d, V, K, loss_mask


def _workspace(workspace, N, d, V, K, chunk, dt, dev, dw_group_tokens=None):
    import torch
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(N, d, V, K, chunk, dt, dw_group_tokens), 256),
                                dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, dev)
    return workspace


def _check_workspace(workspace, dev):
    import torch
    _on_device(dev, workspace=workspace)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


def _stream(stream, dev):
    import torch
    return torch.cuda.current_stream(dev).cuda_stream if stream is None else stream


def fwd_bwd(h, W, topk_idx, topk_p, loss_mask=None, chunk: int = 2048, rows: bool = False,
            workspace=None, stream=None, dw_group_tokens: Optional[int] = None,
            dh_float32: bool = False):
    """Mean top-K KL loss with its gradients, computed chunk by chunk on the GPU.

    Args (torch CUDA tensors, contiguous):
      h [N, d] and W [V, d]: bfloat16 or float32 (same dtype);
      topk_idx [N, K] int32; topk_p [N, K] float32; loss_mask [N] uint8/bool or None.
      chunk: token rows whose logits are live at once.
      rows: also return per-row loss, logsumexp and the logits at the teacher's indices.
      workspace: optional uint8 tensor; the call takes the largest dW group it holds.
      dw_group_tokens: size of the workspace allocated when none is given (see
        ``workspace_bytes``); None is the default, full-speed group.
      dh_float32: return dh as the float32 sums, not rounded to h's dtype
        (kd_chunked_kl_fwd_bwd_f32dh), e.g. for ``scale_grads``.
    Returns (loss[1] f32, dh [N, d] dtype, dW [V, d] f32) and, with ``rows``,
    (row_loss [N], row_lse [N], zg [N, K]) as float32.
    """
    import torch
    dt, N, d, V, K, loss_mask = _prep(h, W, topk_idx, topk_p, loss_mask)
    dev = h.device
    workspace = _workspace(workspace, N, d, V, K, chunk, dt, dev, dw_group_tokens)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    dh = torch.empty((N, d), dtype=torch.float32 if dh_float32 else h.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    row_loss = row_lse = zg = None
    if rows:
        row_loss = torch.empty(N, dtype=torch.float32, device=dev)
        row_lse = torch.empty(N, dtype=torch.float32, device=dev)
        zg = torch.empty((N, K), dtype=torch.float32, device=dev)
    call = _lib().kd_chunked_kl_fwd_bwd_f32dh if dh_float32 else _lib().kd_chunked_kl_fwd_bwd
    _check(call(
        _ptr(h), _ptr(W), dt, _ptr(topk_idx), _ptr(topk_p), _ptr(loss_mask), N, d, V, K, chunk,
        _ptr(loss), _ptr(dh), _ptr(dW), _ptr(row_loss), _ptr(row_lse), _ptr(zg),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    if rows:
        return loss, dh, dW, row_loss, row_lse, zg
    return loss, dh, dW


def fwd_bwd_async(h, W, topk_idx, topk_p, loss_mask, loss, dh, dW, status, workspace,
                  chunk: int = 2048, row_loss=None, row_lse=None, zg=None, stream=None) -> None:
    """kd_chunked_kl_fwd_bwd_async: the one-call loss into caller-given outputs with no host
    synchronisation, so that it can be recorded into a graph (torch.cuda.graph) and
    replayed.  Outputs as ``fwd_bwd`` returns them (loss [1] f32, dh [N, d] h's dtype,
    dW [V, d] f32, optional row outputs); ``status`` is a [1] int32 CUDA tensor set to 0,
    or to 2 (KD_E_INDEX) when a teacher entry is invalid (then the outputs are undefined).
    ``workspace`` is required (a recorded graph must not allocate)."""
    import torch
    if workspace is None:
        raise ValueError("workspace is required (a recorded graph must not allocate)")
    dt, N, d, V, K, loss_mask = _prep(h, W, topk_idx, topk_p, loss_mask)
    dev = h.device
    _on_device(dev, loss=loss, dh=dh, dW=dW, status=status, row_loss=row_loss,
               row_lse=row_lse, zg=zg)
    _check_workspace(workspace, dev)
    want = [(loss, (1,), torch.float32), (dh, (N, d), h.dtype), (dW, (V, d), torch.float32),
            (status, (1,), torch.int32), (row_loss, (N,), torch.float32),
            (row_lse, (N,), torch.float32), (zg, (N, K), torch.float32)]
    for t, shape, dtype in want:
        if t is not None and (tuple(t.shape) != shape or t.dtype != dtype
                              or not t.is_contiguous()):
            raise ValueError(f"an output has shape {tuple(t.shape)} and dtype {t.dtype}; "
                             f"expected contiguous {shape} {dtype}")
    _check(_lib().kd_chunked_kl_fwd_bwd_async(
        _ptr(h), _ptr(W), dt, _ptr(topk_idx), _ptr(topk_p), _ptr(loss_mask), N, d, V, K, chunk,
        _ptr(loss), _ptr(dh), _ptr(dW), _ptr(row_loss), _ptr(row_lse), _ptr(zg), _ptr(status),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))


def fwd(h, W, topk_idx, topk_p, loss_mask=None, chunk: int = 2048, rows: bool = False,
        workspace=None, stream=None):
    """Forward half: (loss[1] f32, row_lse [N] f32) and, with ``rows``, also
    (row_loss [N], zg [N, K]).  row_lse is the state ``bwd`` needs."""
    import torch
    dt, N, d, V, K, loss_mask = _prep(h, W, topk_idx, topk_p, loss_mask)
    dev = h.device
    workspace = _workspace(workspace, N, d, V, K, chunk, dt, dev, 0)  # no dW group
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_loss = zg = None
    if rows:
        row_loss = torch.empty(N, dtype=torch.float32, device=dev)
        zg = torch.empty((N, K), dtype=torch.float32, device=dev)
    _check(_lib().kd_chunked_kl_fwd(
        _ptr(h), _ptr(W), dt, _ptr(topk_idx), _ptr(topk_p), _ptr(loss_mask), N, d, V, K, chunk,
        _ptr(loss), _ptr(row_lse), _ptr(row_loss), _ptr(zg), _ptr(workspace), workspace.numel(),
        _stream(stream, dev)))
    if rows:
        return loss, row_lse, row_loss, zg
    return loss, row_lse


def bwd(h, W, topk_idx, topk_p, row_lse, grad_loss=None, loss_mask=None, chunk: int = 2048,
        workspace=None, stream=None, dw_group_tokens: Optional[int] = None):
    """Backward half: (dh [N, d] dtype, dW [V, d] f32) for the upstream gradient
    ``grad_loss`` (a one-element float32 CUDA tensor; None means 1), recomputing the
    logits from h and W with the ``row_lse`` saved by ``fwd``.  ``workspace`` and
    ``dw_group_tokens`` as in ``fwd_bwd``."""
    import torch
    dt, N, d, V, K, loss_mask = _prep(h, W, topk_idx, topk_p, loss_mask)
    dev = h.device
    _on_device(dev, row_lse=row_lse, grad_loss=grad_loss)
    if row_lse.dtype != torch.float32 or tuple(row_lse.shape) != (N,) or not row_lse.is_contiguous():
        raise ValueError("row_lse must be a contiguous float32 tensor of shape [N]")
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
    grad_loss = grad_loss.reshape(1)
    if grad_loss.dtype != torch.float32:
        raise TypeError("grad_loss must be float32")
    grad_loss = grad_loss.contiguous()
    workspace = _workspace(workspace, N, d, V, K, chunk, dt, dev, dw_group_tokens)
    dh = torch.empty((N, d), dtype=h.dtype, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    _check(_lib().kd_chunked_kl_bwd(
        _ptr(h), _ptr(W), dt, _ptr(topk_idx), _ptr(topk_p), _ptr(loss_mask), N, d, V, K, chunk,
        _ptr(row_lse), _ptr(grad_loss), _ptr(dh), _ptr(dW), _ptr(workspace), workspace.numel(),
        _stream(stream, dev)))
    return dh, dW


def scale_grads(grad_loss, dh_f32, dW, dtype=None, stream=None):
    """Gradients for an upstream gradient g of the loss from those for g = 1
    (kd_scale_grads): returns dh = g * dh_f32 rounded once to ``dtype`` (default
    float32) and scales ``dW`` in place (untouched when g == 1), which it also returns."""
    import torch
    dev = dh_f32.device
    _on_device(dev, grad_loss=grad_loss, dh_f32=dh_f32, dW=dW)
    dtype = torch.float32 if dtype is None else dtype
    dt = KD_BF16 if dtype == torch.bfloat16 else KD_F32 if dtype == torch.float32 else None
    if dt is None:
        raise TypeError("dh must be bfloat16 or float32")
    if (dh_f32.dtype != torch.float32 or dW.dtype != torch.float32 or dh_f32.dim() != 2
            or dW.dim() != 2 or dW.shape[1] != dh_f32.shape[1] or not dh_f32.is_contiguous()
            or not dW.is_contiguous()):
        raise ValueError("dh_f32 [N, d] and dW [V, d] must be contiguous float32")
    if grad_loss.dtype != torch.float32 or grad_loss.numel() != 1:
        raise TypeError("grad_loss must be a one-element float32 tensor")
    g = grad_loss.reshape(1).contiguous()
    N, d = dh_f32.shape
    dh = torch.empty((N, d), dtype=dtype, device=dev)
    _check(_lib().kd_scale_grads(_ptr(g), _ptr(dh_f32), _ptr(dh), dt, N, d, _ptr(dW),
                                 dW.shape[0], _stream(stream, dev)))
    return dh, dW


def _autograd_functions():
    import torch

    class ChunkedKLFused(torch.autograd.Function):
        """The loss as an autograd function of h and W at the one-call speed: the forward
        runs the one-call loss and gradients for g = 1 (dh kept in float32) and holds
        them; the backward applies the upstream gradient g on the device."""

        @staticmethod
        def forward(ctx, h, W, topk_idx, topk_p, loss_mask, chunk):
            loss, dh32, dW = fwd_bwd(h, W, topk_idx, topk_p, loss_mask, chunk,
                                     dh_float32=True)
            ctx.grads = (dh32, dW)
            ctx.h_dtype = h.dtype
            return loss.view(())

        @staticmethod
        def backward(ctx, grad_out):
            if ctx.grads is None:
                raise RuntimeError("the fused chunked KL loss can be differentiated once; "
                                   "use mode='recompute' to call backward again")
            dh32, dW = ctx.grads
            ctx.grads = None
            g = grad_out.detach().reshape(1).to(torch.float32).contiguous()
            dh, dW = scale_grads(g, dh32, dW, ctx.h_dtype)
            del dh32
            # dW is float32; autograd converts it to W's dtype if they differ
            return dh, dW, None, None, None, None

    class ChunkedKL(torch.autograd.Function):
        """The loss as an autograd function of h and W: the forward keeps only the
        per-token logsumexp; the backward recomputes the logits chunk by chunk."""

        @staticmethod
        def forward(ctx, h, W, topk_idx, topk_p, loss_mask, chunk):
            loss, row_lse = fwd(h, W, topk_idx, topk_p, loss_mask, chunk)
            ctx.save_for_backward(h, W, topk_idx, topk_p, loss_mask, row_lse)
            ctx.chunk = chunk
            return loss.view(())

        @staticmethod
        def backward(ctx, grad_out):
            h, W, topk_idx, topk_p, loss_mask, row_lse = ctx.saved_tensors
            g = grad_out.detach().reshape(1).to(torch.float32).contiguous()
            dh, dW = bwd(h, W, topk_idx, topk_p, row_lse, g, loss_mask, ctx.chunk)
            # dW is float32; autograd converts it to W's dtype if they differ
            return dh, dW, None, None, None, None

    return {"fused": ChunkedKLFused, "recompute": ChunkedKL}


_CHUNKED_KL = None


def chunked_kl_loss(h, W, topk_idx, topk_p, loss_mask=None, chunk: int = 2048,
                    mode: str = "fused"):
    """Mean top-K KL loss as a differentiable scalar of h and W (torch autograd).

    mode "fused" (default): the forward computes the loss and both gradients in one
      call and holds dh (float32) and dW until the backward, which scales them by the
      upstream gradient on the device: the one-call speed, with those two tensors
      alive between forward and backward.  Differentiable once.
    mode "recompute": the forward keeps only the per-token logsumexp; the backward
      recomputes the logits chunk by chunk (the pages' autograd form)."""
    global _CHUNKED_KL
    if _CHUNKED_KL is None:
        _CHUNKED_KL = _autograd_functions()
    if mode not in _CHUNKED_KL:
        raise ValueError(f"mode must be 'fused' or 'recompute', not {mode!r}")
    return _CHUNKED_KL[mode].apply(h, W, topk_idx, topk_p, loss_mask, chunk)


def teacher_topk(logits, K: int = 100, lse: bool = True, workspace=None, stream=None):
    """Teacher top-K cache for ``logits`` [N, V] (bfloat16 or float32 CUDA tensor):
    ``(topk_idx [N, K] int32, topk_p [N, K] float32[, row_lse [N] float32])``."""
    import torch
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [N, V] tensor")
    dt = _dtype_code(logits)
    N, V = logits.shape
    dev = logits.device
    _on_device(dev, logits=logits)
    if workspace is None:
        out = ctypes.c_size_t(0)
        _check(_lib().kd_topk_workspace_bytes(ctypes.byref(out)))
        workspace = torch.empty(int(out.value), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, dev)
    idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    p = torch.empty((N, K), dtype=torch.float32, device=dev)
    row_lse = torch.empty(N, dtype=torch.float32, device=dev) if lse else None
    _check(_lib().kd_teacher_topk(_ptr(logits), dt, N, V, K, _ptr(idx), _ptr(p), _ptr(row_lse),
                                  _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return (idx, p, row_lse) if lse else (idx, p)


def vocab_shard_fwd(h, W_shard, topk_idx, topk_p, v_offset: int, V_total: int,
                    chunk: int = 2048, zg: bool = False, workspace=None, stream=None):
    """One vocabulary shard's forward statistics: ``(shard_max, shard_sumexp, shard_pz)``
    [N] float32 each (and zg [N, K] with ``zg``)."""
    import torch
    dt, N, d, Vs, K, _ = _prep(h, W_shard, topk_idx, topk_p, None)
    dev = h.device
    workspace = _workspace(workspace, N, d, Vs, K, chunk, dt, dev, 0)  # no dW group
    st = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3)]
    zgt = torch.empty((N, K), dtype=torch.float32, device=dev) if zg else None
    _check(_lib().kd_vocab_shard_fwd(
        _ptr(h), _ptr(W_shard), dt, _ptr(topk_idx), _ptr(topk_p), N, d, Vs, v_offset, V_total, K,
        chunk, _ptr(st[0]), _ptr(st[1]), _ptr(st[2]), _ptr(zgt), _ptr(workspace),
        workspace.numel(), _stream(stream, h.device)))
    return (*st, zgt) if zg else tuple(st)


def vocab_shard_combine(shard_max, shard_sumexp, shard_pz, topk_p, loss_mask=None,
                        workspace=None, stream=None):
    """Global ``(loss[1], row_lse [N], row_loss [N])`` from G shards' statistics, each
    given as a [G, N] float32 tensor."""
    import torch
    G, N = shard_max.shape
    K = topk_p.shape[1]
    dev = shard_max.device
    _on_device(dev, shard_max=shard_max, shard_sumexp=shard_sumexp, shard_pz=shard_pz,
               topk_p=topk_p, loss_mask=loss_mask)
    for t in (shard_max, shard_sumexp, shard_pz, topk_p):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("shard statistics and topk_p must be contiguous float32")
    if (tuple(shard_sumexp.shape) != (G, N) or tuple(shard_pz.shape) != (G, N)
            or topk_p.dim() != 2 or topk_p.shape[0] != N):
        raise ValueError("shard statistics must be [G, N] and topk_p [N, K]")
    if loss_mask is not None:
        if loss_mask.dtype == torch.bool:
            loss_mask = loss_mask.view(torch.uint8)
        if (loss_mask.dtype != torch.uint8 or tuple(loss_mask.shape) != (N,)
                or not loss_mask.is_contiguous()):
            raise ValueError("loss_mask must be contiguous uint8/bool of shape [N]")
    if workspace is None:
        out = ctypes.c_size_t(0)
        _check(_lib().kd_vocab_shard_combine_workspace_bytes(N, ctypes.byref(out)))
        workspace = torch.empty(int(out.value), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_loss = torch.empty(N, dtype=torch.float32, device=dev)
    _check(_lib().kd_vocab_shard_combine(
        _ptr(shard_max), _ptr(shard_sumexp), _ptr(shard_pz), G, _ptr(topk_p), _ptr(loss_mask), N,
        K, _ptr(loss), _ptr(row_lse), _ptr(row_loss), _ptr(workspace), workspace.numel(),
        _stream(stream, dev)))
    return loss, row_lse, row_loss


def vocab_shard_bwd(h, W_shard, topk_idx, topk_p, row_lse, v_offset: int, V_total: int,
                    grad_loss=None, loss_mask=None, chunk: int = 2048, workspace=None,
                    stream=None):
    """One shard's ``(dh_partial [N, d] float32, dW_shard [V_shard, d] float32)``."""
    import torch
    dt, N, d, Vs, K, loss_mask = _prep(h, W_shard, topk_idx, topk_p, loss_mask)
    dev = h.device
    _on_device(dev, row_lse=row_lse, grad_loss=grad_loss)
    if row_lse.dtype != torch.float32 or tuple(row_lse.shape) != (N,) or not row_lse.is_contiguous():
        raise ValueError("row_lse must be a contiguous float32 tensor of shape [N]")
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
    if grad_loss.dtype != torch.float32 or grad_loss.numel() != 1:
        raise TypeError("grad_loss must be a one-element float32 tensor")
    grad_loss = grad_loss.reshape(1).contiguous()
    workspace = _workspace(workspace, N, d, Vs, K, chunk, dt, dev)
    dh = torch.empty((N, d), dtype=torch.float32, device=dev)
    dW = torch.empty((Vs, d), dtype=torch.float32, device=dev)
    _check(_lib().kd_vocab_shard_bwd(
        _ptr(h), _ptr(W_shard), dt, _ptr(topk_idx), _ptr(topk_p), _ptr(loss_mask), N, d, Vs,
        v_offset, V_total, K, chunk, _ptr(row_lse), _ptr(grad_loss), _ptr(dh), _ptr(dW),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return dh, dW


def profile_enable(on: bool = True) -> None:
    _check(_lib().kd_profile_enable(1 if on else 0))


def profile_classes():
    lib = _lib()
    return [lib.kd_profile_class_name(i).decode() for i in range(lib.kd_profile_num_classes())]


def clock_stamp(stamps, stream=None) -> None:
    """Enqueues kd_clock_stamp into ``stamps``, a contiguous int64 CUDA tensor of
    3 * n_groups elements (per workgroup: compute unit, its cycle counter, the constant
    counter)."""
    import torch
    if stamps.dtype != torch.int64 or not stamps.is_contiguous() or stamps.numel() % 3:
        raise ValueError("stamps must be a contiguous int64 tensor of 3 * n_groups elements")
    _on_device(stamps.device, stamps=stamps)
    _check(_lib().kd_clock_stamp(_ptr(stamps), stamps.numel() // 3,
                                 _stream(stream, stamps.device)))


def wall_clock_khz() -> int:
    """Rate of the constant counter that kd_clock_stamp records, in kHz."""
    out = ctypes.c_int32(0)
    _check(_lib().kd_wall_clock_khz(ctypes.byref(out)))
    return int(out.value)


def profile_read():
    """{class name: (total_ms, launches)} for launches since the last read (waits for them)."""
    lib = _lib()
    out = {}
    for i, name in enumerate(profile_classes()):
        ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(lib.kd_profile_read(i, ctypes.byref(ms), ctypes.byref(n)))
        out[name] = (ms.value, n.value)
    return out
