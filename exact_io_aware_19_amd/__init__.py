"""Exact IO-aware attention for AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI in include/fa.h (libfa355.so).  Every step of the
computation runs in the library's HIP kernels; this module only marshals torch tensors
(device memory and the current stream) into the C calls.  There is no fallback path:
if the library is missing or a call fails, an exception is raised.

Low-level calls with the C names (caller allocates every output):
    fa_forward(q, k, v, o, lse, scale, causal, kv_len=None, stream=None)
    fa_backward(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                kv_len=None, stream=None)
    fa_backward_workspace_size(B, H, N, d)
    fa_backward_pass(which, ...)  # "dq" or "dkdv": the two passes of fa_backward
    fa_forward_gqa(q, k, v, o, lse, scale, causal, kv_len=None, stream=None)
    fa_backward_gqa(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                    kv_len=None, stream=None)
    fa_backward_gqa_workspace_size(B, H, H_kv, N, d)
        grouped K/V heads: k, v, dk, dv are [B, H_kv, N, d] with H_kv dividing H

Convenience wrappers that allocate outputs with torch (grouped K/V heads when k has
fewer heads than q):
    forward(q, k, v, causal=False, scale=None, kv_len=None) -> (o, lse)
    backward(q, k, v, o, dout, lse, causal=False, scale=None, kv_len=None) -> (dq, dk, dv)

Tensors: q, k, v, o, dout, dq, dk, dv are contiguous bf16 [B, H, N, d] on the GPU
(d in {64, 128}); lse is fp32 [B, H, N]; kv_len is int32 [B] on the GPU.
"""

import math

from . import _lib

__all__ = [
    "fa_forward",
    "fa_backward",
    "fa_backward_workspace_size",
    "fa_backward_pass",
    "fa_forward_gqa",
    "fa_backward_gqa",
    "fa_backward_gqa_workspace_size",
    "forward",
    "backward",
    "FAError",
]

FAError = _lib.FAError


def _torch():
    import torch

    return torch


def _check_qkv(name, t, shape=None):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_lse(t, shape):
    torch = _torch()
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape[:3]) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"lse must be a contiguous fp32 GPU tensor of shape {tuple(shape[:3])}")


def _kv_ptr(kv_len, B, device):
    torch = _torch()
    if kv_len is None:
        return None
    if kv_len.dtype != torch.int32 or kv_len.dim() != 1 or kv_len.numel() != B or not kv_len.is_cuda:
        raise ValueError("kv_len must be an int32 GPU tensor of shape [B]")
    if kv_len.device != device:
        raise ValueError("kv_len must live on the same device as q")
    return kv_len.contiguous().data_ptr()


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def fa_forward(q, k, v, o, lse, scale, causal, kv_len=None, stream=None):
    """C ``fa_forward`` / ``fa_forward_kvlen``: fills o (bf16) and lse (fp32) in place."""
    _check_qkv("q", q)
    shape = tuple(q.shape)
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check_qkv(name, t, shape)
    _check_lse(lse, shape)
    B, H, N, d = shape
    lib = _lib.load()
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    if kvp is None:
        st = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                            float(scale), int(bool(causal)), sp)
        _lib.check(st, "fa_forward")
    else:
        st = lib.fa_forward_kvlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                                  d, float(scale), int(bool(causal)), kvp, sp)
        _lib.check(st, "fa_forward_kvlen")


def _kv_shape(q, k):
    """[B, H_kv, N, d] of grouped K/V heads for q of shape [B, H, N, d]."""
    B, H, N, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, H_kv, {N}, {d}]")
    hkv = int(k.shape[1])
    if hkv < 1 or H % hkv:
        raise ValueError(f"K/V heads ({hkv}) must divide query heads ({H})")
    return (B, hkv, N, d)


def fa_forward_gqa(q, k, v, o, lse, scale, causal, kv_len=None, stream=None):
    """C ``fa_forward_gqa``: k, v are [B, H_kv, N, d]; fills o and lse in place."""
    _check_qkv("q", q)
    shape = tuple(q.shape)
    kv_shape = _kv_shape(q, k)
    _check_qkv("k", k, kv_shape)
    _check_qkv("v", v, kv_shape)
    _check_qkv("o", o, shape)
    _check_lse(lse, shape)
    B, H, N, d = shape
    lib = _lib.load()
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    st = lib.fa_forward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                            kv_shape[1], N, d, float(scale), int(bool(causal)), kvp, sp)
    _lib.check(st, "fa_forward_gqa")


def fa_backward_gqa(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len=None, stream=None):
    """C ``fa_backward_gqa``: k, v, dk, dv are [B, H_kv, N, d]; fills dq, dk, dv in place.

    workspace: a GPU tensor of at least fa_backward_gqa_workspace_size(B, H, H_kv, N, d) bytes.
    """
    _check_qkv("q", q)
    shape = tuple(q.shape)
    kv_shape = _kv_shape(q, k)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _check_qkv(name, t, kv_shape)
    for name, t in (("o", o), ("dout", dout), ("dq", dq)):
        _check_qkv(name, t, shape)
    _check_lse(lse, shape)
    B, H, N, d = shape
    lib = _lib.load()
    nbytes = workspace.numel() * workspace.element_size()
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    st = lib.fa_backward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, kv_shape[1], N, d, float(scale),
                             int(bool(causal)), kvp, workspace.data_ptr(), nbytes, sp)
    _lib.check(st, "fa_backward_gqa")


def fa_backward_workspace_size(B, H, N, d):
    """C ``fa_backward_workspace_size``."""
    return int(_lib.load().fa_backward_workspace_size(B, H, N, d))


def fa_backward_gqa_workspace_size(B, H, H_kv, N, d):
    """C ``fa_backward_gqa_workspace_size``."""
    return int(_lib.load().fa_backward_gqa_workspace_size(B, H, H_kv, N, d))


def fa_backward(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len=None, stream=None):
    """C ``fa_backward`` / ``fa_backward_kvlen``: fills dq, dk, dv (bf16) in place.

    workspace: a GPU tensor (any dtype) of at least fa_backward_workspace_size bytes.
    """
    _backward_call(None, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len, stream)


def fa_backward_pass(which, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len=None, stream=None):
    """C ``fa_backward_dq_pass`` (which="dq") or ``fa_backward_dkdv_pass`` (which="dkdv").

    The two passes in that order on one stream are exactly ``fa_backward``.
    """
    if which not in ("dq", "dkdv"):
        raise ValueError("which must be 'dq' or 'dkdv'")
    _backward_call(which, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len, stream)


def _backward_call(which, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace, kv_len, stream):
    _check_qkv("q", q)
    shape = tuple(q.shape)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_qkv(name, t, shape)
    _check_lse(lse, shape)
    B, H, N, d = shape
    lib = _lib.load()
    nbytes = workspace.numel() * workspace.element_size()
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal))]
    if which is not None:
        name = f"fa_backward_{which}_pass"
        st = getattr(lib, name)(*args, kvp, workspace.data_ptr(), nbytes, sp)
        _lib.check(st, name)
    elif kvp is None:
        st = lib.fa_backward(*args, workspace.data_ptr(), nbytes, sp)
        _lib.check(st, "fa_backward")
    else:
        st = lib.fa_backward_kvlen(*args, kvp, workspace.data_ptr(), nbytes, sp)
        _lib.check(st, "fa_backward_kvlen")


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal=False, scale=None, kv_len=None):
    """Allocate o and lse, run the fused forward; returns (o, lse)."""
    torch = _torch()
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if k.dim() == 4 and k.shape[1] != H:
        fa_forward_gqa(q, k, v, o, lse, _default_scale(d, scale), causal, kv_len=kv_len)
    else:
        fa_forward(q, k, v, o, lse, _default_scale(d, scale), causal, kv_len=kv_len)
    return o, lse


def backward(q, k, v, o, dout, lse, causal=False, scale=None, kv_len=None, workspace=None):
    """Allocate dq, dk, dv (and a workspace unless given), run the backward."""
    torch = _torch()
    B, H, N, d = q.shape
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    grouped = k.dim() == 4 and k.shape[1] != H
    if workspace is None:
        nbytes = (fa_backward_gqa_workspace_size(B, H, int(k.shape[1]), N, d) if grouped
                  else fa_backward_workspace_size(B, H, N, d))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if grouped:
        fa_backward_gqa(q, k, v, o, dout, lse, dq, dk, dv, _default_scale(d, scale), causal, workspace,
                        kv_len=kv_len)
    else:
        fa_backward(q, k, v, o, dout, lse, dq, dk, dv, _default_scale(d, scale), causal, workspace, kv_len=kv_len)
    return dq, dk, dv
