"""lm_head_kl_amd: the fused chunked top-K KL distillation loss over the LM head on MI355X.

Python binding of libkdkl (include/kdkl.h). This layer only marshals arguments. PyTorch
supplies device memory (outputs and workspace come from torch.empty on the inputs' device)
and the current HIP stream. Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback.

The loss is a drop-in KL term for a distillation loop: hidden states and the LM-head weight
go in, the offline top-K teacher cache is the target. Source: "Making knowledge distillation
cheap enough to run in production" (aiexpert.news), paragraphs on the two fixes and on the
integration surface.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (KD_ACCUMULATE_DW, KD_BF16, KD_FP32, KD_LOW_MEMORY, KD_SKIP_DW, KD_VALIDATE_IDX, KdError,
                   KdProblem)

__all__ = [
    "FusedKL",
    "fused_kl",
    "fused_kl_fwd",
    "fused_kl_fwd_noalloc",
    "fused_kl_bwd",
    "dense_kl",
    "chunked_kl",
    "chunked_logits",
    "fused_kl_fwdbwd",
    "topk_cache",
    "validate_ids",
    "fused_workspace_bytes",
    "dense_workspace_bytes",
    "chunked_workspace_bytes",
    "fused_fwdbwd_workspace_bytes",
    "make_problem",
    "timing_enable",
    "timing_read",
    "timing_reset",
    "KdError",
    "KD_VALIDATE_IDX",
    "KD_ACCUMULATE_DW",
    "KD_SKIP_DW",
    "KD_LOW_MEMORY",
]

_DT = {torch.bfloat16: KD_BF16, torch.float32: KD_FP32}


def make_problem(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor, tlog: torch.Tensor, T: float,
                 chunk: int, n_norm: float = 0.0, flags: int = 0) -> KdProblem:
    if H.dtype not in _DT or W.dtype != H.dtype:
        raise KdError(3, "make_problem", "H and W must both be bfloat16 or both float32")
    if tlog.dtype not in _DT:
        raise KdError(3, "make_problem", "teacher logits must be bfloat16 or float32")
    if idx.dtype != torch.int32:
        raise KdError(3, "make_problem", "idx must be int32")
    if H.dim() != 2 or W.dim() != 2 or idx.dim() != 2 or tlog.dim() != 2:
        raise KdError(2, "make_problem", "H, W, idx and the teacher logits must be 2-D")
    N, d = H.shape
    V, d2 = W.shape
    if d2 != d or tuple(idx.shape) != tuple(tlog.shape) or idx.shape[0] != N:
        raise KdError(2, "make_problem", f"shape mismatch H{tuple(H.shape)} W{tuple(W.shape)} "
                                         f"idx{tuple(idx.shape)} t{tuple(tlog.shape)}")
    return KdProblem(N=N, d=d, V=V, K=idx.shape[1], chunk=int(chunk), T=float(T), n_norm=float(n_norm),
                     act=_DT[H.dtype], tlogit=_DT[tlog.dtype], flags=int(flags), reserved=0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_device(*ts):
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda" or t.device != dev:
            raise KdError(1, "lm_head_kl_amd", "all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise KdError(2, "lm_head_kl_amd", "tensors must be contiguous (row-major)")
    return dev


def fused_workspace_bytes(p: KdProblem) -> int:
    return int(_lib.lib().kd_fused_workspace_bytes(ctypes.byref(p)))


def dense_workspace_bytes(p: KdProblem) -> int:
    return int(_lib.lib().kd_dense_workspace_bytes(ctypes.byref(p)))


def _workspace(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def _take_workspace(workspace, nbytes: int, dev, where: str):
    """(tensor, size in bytes): the caller's workspace after checks, or a new one. A caller who
    passes one means to avoid an allocation, so one that is too small is an error, not a cue to
    allocate."""
    if workspace is None:
        ws = _workspace(nbytes, dev)
        return ws, ws.numel()
    _need_device(workspace)
    if workspace.device != dev:
        raise KdError(1, where, "the workspace must be on the inputs' GPU")
    size = workspace.numel() * workspace.element_size()
    if size < nbytes:
        raise KdError(5, where, f"workspace holds {size} bytes, the call needs {nbytes}")
    return workspace, size


def _check_dw(dW, W, dev, where: str):
    if dW.dtype != torch.float32 or tuple(dW.shape) != tuple(W.shape):
        raise KdError(3, where, "dW must be float32 with W's shape")
    _need_device(dW)
    if dW.device != dev:
        raise KdError(1, where, "dW must be on the inputs' GPU")


@dataclass
class FwdOut:
    loss: torch.Tensor    # [] fp32
    lse: torch.Tensor     # [N] fp32
    row_kl: torch.Tensor  # [N] fp32 or None
    zk: torch.Tensor      # [N,K] fp32 or None


def fused_kl_fwd(H, W, idx, tlog, T: float = 1.0, chunk: int = 2048, n_norm: float = 0.0,
                 flags: int = 0, want_row_kl: bool = True, want_zk: bool = False,
                 workspace: torch.Tensor | None = None) -> FwdOut:
    """kd_fused_kl_fwd. Returns loss (0-d), lse [N], and optionally row_kl [N] and zk [N,K]."""
    dev = _need_device(H, W, idx, tlog)
    p = make_problem(H, W, idx, tlog, T, chunk, n_norm, flags)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(p.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(p.N, dtype=torch.float32, device=dev) if want_row_kl else None
    zk = torch.empty((p.N, p.K), dtype=torch.float32, device=dev) if want_zk else None
    ws, ws_bytes = _take_workspace(workspace, fused_workspace_bytes(p), dev, "fused_kl_fwd")
    code = _lib.lib().kd_fused_kl_fwd(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlog), _ptr(loss),
                                      _ptr(lse), _ptr(row_kl), _ptr(zk), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(code, "kd_fused_kl_fwd")
    return FwdOut(loss, lse, row_kl, zk)


def fused_kl_fwd_noalloc(H, W, idx, tlog, loss, lse, row_kl=None, zk=None, T: float = 1.0, chunk: int = 2048,
                         n_norm: float = 0.0, flags: int = 0) -> None:
    """kd_fused_kl_fwd_noalloc: the fused forward into caller-owned outputs (loss [] fp32,
    lse [N] fp32, optionally row_kl [N] and zk [N,K] fp32), with the library's static device
    scratch as its workspace. Neither this binding nor the library allocates device memory."""
    dev = _need_device(H, W, idx, tlog, loss, lse, row_kl, zk)
    p = make_problem(H, W, idx, tlog, T, chunk, n_norm, flags)
    for name, t, shape in (("loss", loss, ()), ("lse", lse, (p.N,)), ("row_kl", row_kl, (p.N,)),
                           ("zk", zk, (p.N, p.K))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape):
            raise KdError(3, "fused_kl_fwd_noalloc", f"{name} must be float32 of shape {shape}")
    code = _lib.lib().kd_fused_kl_fwd_noalloc(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlog), _ptr(loss),
                                              _ptr(lse), _ptr(row_kl), _ptr(zk), _stream(dev))
    _lib.check(code, "kd_fused_kl_fwd_noalloc")


def fused_kl_bwd(H, W, idx, tlog, lse, grad_loss=None, T: float = 1.0, chunk: int = 2048,
                 n_norm: float = 0.0, flags: int = 0, dW: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """kd_fused_kl_bwd. Returns (dH [N,d] in H's dtype, dW [V,d] fp32). grad_loss is a device
    scalar tensor or None (= 1). With KD_ACCUMULATE_DW, pass dW to add into. With KD_SKIP_DW
    only dH is computed and dW is returned as None."""
    dev = _need_device(H, W, idx, tlog, lse)
    p = make_problem(H, W, idx, tlog, T, chunk, n_norm, flags)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (p.N,):
        raise KdError(3, "fused_kl_bwd", "lse must be float32 [N], as the forward returns it")
    dH = torch.empty_like(H)
    if flags & KD_SKIP_DW:
        dW = None
    elif dW is None:
        if flags & KD_ACCUMULATE_DW:
            raise KdError(1, "fused_kl_bwd", "KD_ACCUMULATE_DW needs a dW tensor")
        dW = torch.empty(W.shape, dtype=torch.float32, device=dev)
    else:
        _check_dw(dW, W, dev, "fused_kl_bwd")
    g = None
    if grad_loss is not None:
        g = grad_loss.detach().to(device=dev, dtype=torch.float32).reshape(1).contiguous()
    ws, ws_bytes = _take_workspace(workspace, fused_workspace_bytes(p), dev, "fused_kl_bwd")
    code = _lib.lib().kd_fused_kl_bwd(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlog), _ptr(lse),
                                      _ptr(g), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(code, "kd_fused_kl_bwd")
    return dH, dW


def dense_kl(H, W, idx, tlog, T: float = 1.0, grad_loss=None, n_norm: float = 0.0, flags: int = 0,
             want_row_kl: bool = True):
    """kd_dense_kl: loss, lse, row_kl, dH, dW through two dense [N, V] grids."""
    dev = _need_device(H, W, idx, tlog)
    p = make_problem(H, W, idx, tlog, T, 1, n_norm, flags)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(p.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(p.N, dtype=torch.float32, device=dev) if want_row_kl else None
    dH = torch.empty_like(H)
    dW = torch.empty(W.shape, dtype=torch.float32, device=dev)
    g = None
    if grad_loss is not None:
        g = grad_loss.detach().to(device=dev, dtype=torch.float32).reshape(1).contiguous()
    ws = _workspace(dense_workspace_bytes(p), dev)
    code = _lib.lib().kd_dense_kl(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlog), _ptr(g), _ptr(loss),
                                  _ptr(lse), _ptr(row_kl), _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(),
                                  _stream(dev))
    _lib.check(code, "kd_dense_kl")
    return loss, lse, row_kl, dH, dW


def _one_call(fn_name: str, ws_name: str, H, W, idx, tlog, T, chunk, grad_loss, n_norm, flags, want_row_kl, dW,
              workspace):
    dev = _need_device(H, W, idx, tlog)
    p = make_problem(H, W, idx, tlog, T, chunk, n_norm, flags)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(p.N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(p.N, dtype=torch.float32, device=dev) if want_row_kl else None
    dH = torch.empty_like(H)
    if dW is None:
        if flags & KD_ACCUMULATE_DW:
            raise KdError(1, fn_name, "KD_ACCUMULATE_DW needs a dW tensor")
        dW = torch.empty(W.shape, dtype=torch.float32, device=dev)
    else:
        _check_dw(dW, W, dev, fn_name)
    g = None
    if grad_loss is not None:
        g = grad_loss.detach().to(device=dev, dtype=torch.float32).reshape(1).contiguous()
    L = _lib.lib()
    ws, ws_bytes = _take_workspace(workspace, int(getattr(L, ws_name)(ctypes.byref(p))), dev, fn_name)
    code = getattr(L, fn_name)(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(idx), _ptr(tlog), _ptr(g), _ptr(loss),
                               _ptr(lse), _ptr(row_kl), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(code, fn_name)
    return loss, lse, row_kl, dH, dW


def chunked_workspace_bytes(p: KdProblem) -> int:
    return int(_lib.lib().kd_chunked_workspace_bytes(ctypes.byref(p)))


def chunked_logits(p: KdProblem, workspace: torch.Tensor) -> torch.Tensor:
    """kd_chunked_logits: the student logits that kd_chunked_kl keeps, as a view of its
    workspace: z^T [Vp, ldzt] fp32 (Vp = V rounded up to 256), element (v, n) = z[n, v]. Valid
    once the kd_chunked_kl call that used this workspace has run, until the workspace is reused."""
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise KdError(3, "chunked_logits", "the workspace must be a contiguous uint8 tensor")
    zp, ld = ctypes.c_void_p(0), ctypes.c_int64(0)
    code = _lib.lib().kd_chunked_logits(ctypes.byref(p), _ptr(workspace), workspace.numel(), ctypes.byref(zp),
                                        ctypes.byref(ld))
    _lib.check(code, "kd_chunked_logits")
    vp = (p.V + 255) // 256 * 256
    off = int(zp.value) - workspace.data_ptr()
    return workspace[off:off + vp * ld.value * 4].view(torch.float32).view(vp, ld.value)


def fused_fwdbwd_workspace_bytes(p: KdProblem) -> int:
    return int(_lib.lib().kd_fused_fwdbwd_workspace_bytes(ctypes.byref(p)))


def chunked_kl(H, W, idx, tlog, T: float = 1.0, chunk: int = 2048, grad_loss=None, n_norm: float = 0.0,
               flags: int = 0, want_row_kl: bool = True, dW=None, workspace=None):
    """kd_chunked_kl (forward-chunked formulation: every logit kept for the backward).
    Returns (loss, lse, row_kl, dH, dW)."""
    return _one_call("kd_chunked_kl", "kd_chunked_workspace_bytes", H, W, idx, tlog, T, chunk, grad_loss, n_norm,
                     flags, want_row_kl, dW, workspace)


def fused_kl_fwdbwd(H, W, idx, tlog, T: float = 1.0, chunk: int = 2048, grad_loss=None, n_norm: float = 0.0,
                    flags: int = 0, want_row_kl: bool = True, dW=None, workspace=None):
    """kd_fused_kl_fwdbwd (single pass per chunk, no recompute; grad_loss applied now).
    Returns (loss, lse, row_kl, dH, dW)."""
    return _one_call("kd_fused_kl_fwdbwd", "kd_fused_fwdbwd_workspace_bytes", H, W, idx, tlog, T, chunk, grad_loss,
                     n_norm, flags, want_row_kl, dW, workspace)


def topk_cache(logits: torch.Tensor, K: int):
    """kd_topk_cache: the offline teacher cache. logits [N, V] (bf16 or fp32, rows may be
    strided) -> (idx [N, K] int32, values [N, K] in the logits' dtype), largest first, ties by
    the lower token id."""
    if logits.dtype not in _DT:
        raise KdError(3, "topk_cache", "logits must be bfloat16 or float32")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise KdError(2, "topk_cache", "logits must be [N, V] with contiguous rows")
    N, V = logits.shape
    if not 1 <= int(K) <= min(V, 1024):
        raise KdError(2, "topk_cache", f"K = {K} outside 1 .. min(V, 1024) = {min(V, 1024)}")
    if logits.device.type != "cuda":
        raise KdError(1, "topk_cache", "logits must be on a GPU")
    dev = logits.device
    idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    vals = torch.empty((N, K), dtype=logits.dtype, device=dev)
    code = _lib.lib().kd_topk_cache(_ptr(logits), _DT[logits.dtype], N, V, logits.stride(0), int(K), _ptr(idx),
                                    _ptr(vals), _stream(dev))
    _lib.check(code, "kd_topk_cache")
    return idx, vals


def validate_ids(idx: torch.Tensor, V: int, status: torch.Tensor | None = None) -> torch.Tensor:
    """kd_validate_ids: checks the cached ids without synchronising. Returns the device status
    word (uint32 viewed as int32, one element): 0 if every row holds K distinct ids in [0, V),
    else bit 1 (an id out of range) and/or bit 2 (a repeated id). Pass `status` to reuse one
    word, e.g. inside a captured graph."""
    if idx.dtype != torch.int32 or idx.dim() != 2:
        raise KdError(3, "validate_ids", "idx must be int32 [N, K]")
    dev = _need_device(idx)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    elif status.dtype != torch.int32 or status.numel() < 1 or status.device != dev or not status.is_contiguous():
        raise KdError(3, "validate_ids", "status must be a contiguous int32 tensor on idx's GPU")
    code = _lib.lib().kd_validate_ids(_ptr(idx), idx.shape[0], idx.shape[1], int(V), _ptr(status), _stream(dev))
    _lib.check(code, "kd_validate_ids")
    return status


class FusedKL(torch.autograd.Function):
    """loss = FusedKL.apply(H, W, idx, tlog, T, chunk, n_norm, dw_accumulator, low_memory): the
    KL term of a distillation step. The forward saves only lse [N]; the backward recomputes the
    logits chunk by chunk.

    dW is always accumulated in fp32 by the library. Without `dw_accumulator` it becomes W's
    gradient in W's dtype (autograd requires that dtype, so a bf16 head receives dW rounded to
    bf16). With `dw_accumulator` (an fp32 tensor of W's shape) the backward adds dW into it
    (KD_ACCUMULATE_DW) and gives W no autograd gradient, so micro-batches sum in fp32 in the
    caller's buffer. A head that needs no gradient and has no accumulator skips the dW work
    (KD_SKIP_DW). `low_memory` selects the memory-lean backward (KD_LOW_MEMORY)."""

    @staticmethod
    def forward(ctx, H, W, idx, tlog, T=1.0, chunk=2048, n_norm=0.0, dw_accumulator=None, low_memory=False):
        out = fused_kl_fwd(H, W, idx, tlog, T=T, chunk=chunk, n_norm=n_norm, want_row_kl=False)
        if dw_accumulator is not None:
            _check_dw(dw_accumulator, W, H.device, "FusedKL")
            if not dw_accumulator.is_contiguous():
                raise KdError(2, "FusedKL", "dw_accumulator must be contiguous")
        ctx.save_for_backward(H, W, idx, tlog, out.lse)
        ctx.cfg = (T, chunk, n_norm, bool(low_memory))
        ctx.dw_acc = dw_accumulator
        return out.loss

    @staticmethod
    def backward(ctx, g):
        H, W, idx, tlog, lse = ctx.saved_tensors
        T, chunk, n_norm, lean = ctx.cfg
        acc = ctx.dw_acc
        flags = KD_LOW_MEMORY if lean else 0
        if acc is not None:
            flags |= KD_ACCUMULATE_DW
        elif not ctx.needs_input_grad[1]:
            flags |= KD_SKIP_DW  # a frozen head skips dW and the work that only it needs
        dH, dW = fused_kl_bwd(H, W, idx, tlog, lse, grad_loss=g, T=T, chunk=chunk, n_norm=n_norm, flags=flags,
                              dW=acc)
        dW_out = dW.to(W.dtype) if (acc is None and dW is not None) else None
        return dH, dW_out, None, None, None, None, None, None, None


def fused_kl(H, W, idx, tlog, T: float = 1.0, chunk: int = 2048, n_norm: float = 0.0,
             dw_accumulator: torch.Tensor | None = None, low_memory: bool = False):
    return FusedKL.apply(H, W, idx, tlog, T, chunk, n_norm, dw_accumulator, low_memory)


def timing_enable(on: bool = True) -> bool:
    """Turn per-kernel HIP-event timing inside the library on or off; returns the old setting."""
    return bool(_lib.lib().kd_timing_enable(1 if on else 0))


def timing_reset() -> None:
    _lib.lib().kd_timing_reset()


def timing_read() -> dict:
    """{kernel kind: (launches, total milliseconds)} accumulated since the last reset (waits for
    the recorded events)."""
    L = _lib.lib()
    out = {}
    for k in range(L.kd_timing_kinds()):
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _lib.check(L.kd_timing_read(k, ctypes.byref(n), ctypes.byref(ms)), "kd_timing_read")
        if n.value:
            out[L.kd_timing_name(k).decode()] = (int(n.value), float(ms.value))
    return out
