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
    fa_backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len=None,
                        stream=None)
        no workspace: the library's own scratch (NOALLOC_SCRATCH_BYTES per GPU); calls
        that overlap on one GPU race
    fa_forward_gqa(q, k, v, o, lse, scale, causal, kv_len=None, stream=None)
    fa_backward_gqa(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                    kv_len=None, stream=None)
    fa_backward_gqa_workspace_size(B, H, H_kv, N, d)
        grouped K/V heads: k, v, dk, dv are [B, H_kv, N, d] with H_kv dividing H
    fa_forward_offset(q, k, v, o, lse, scale, causal, q_offset, kv_len=None, stream=None)
        q, o [B, H, Nq, d] against k, v [B, H, Nk, d]; query row i at key position
        q_offset + i (one GPU's share of a query-split forward)

FP8 forward (block quantisation + incoherent processing; OCP E4M3 codes as uint8):
    fa_fp8_quantize_qk(x, x8, scales, signs=None, post_scale=1.0, stream=None)
        x bf16 [B, H, N, d] -> x8 uint8 [B, H, N, d], scales fp32 [B, H, ceil(N/64)]
    fa_fp8_quantize_v(v, v8t, scales, stream=None)
        v bf16 [B, H, N, d] -> v8t uint8 [B, H, ceil(N/64), d, 64] (transposed tiles in
        the key order of the P V product), scales fp32 [B, H, d]
    fa_forward_fp8(q8, sq, k8, sk, v8t, sv, o, lse, scale, causal, kv_len=None, stream=None)
    fp8_v8t_to_rows(v8t, N): the codes of fa_fp8_quantize_v back in [B, H, N, d] order
    forward_fp8(q, k, v, causal=False, scale=None, kv_len=None, signs=None) -> (o, lse)

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
    "fa_backward_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "fa_forward_gqa",
    "fa_forward_offset",
    "fa_backward_gqa",
    "fa_backward_gqa_workspace_size",
    "fa_fp8_quantize_qk",
    "fa_fp8_quantize_v",
    "fa_forward_fp8",
    "fp8_v8t_to_rows",
    "forward_fp8",
    "forward",
    "backward",
    "FAError",
]

FAError = _lib.FAError
NOALLOC_SCRATCH_BYTES = _lib.NOALLOC_SCRATCH_BYTES


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


def fa_forward_offset(q, k, v, o, lse, scale, causal, q_offset, kv_len=None, stream=None):
    """C ``fa_forward_offset``: q, o [B, H, Nq, d]; k, v [B, H, Nk, d]; query row i sits at
    key position q_offset + i.  Fills o and lse [B, H, Nq] in place."""
    _check_qkv("q", q)
    shape = tuple(q.shape)
    B, H, Nq, d = shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, {H}, Nk, {d}]")
    kv_shape = tuple(k.shape)
    _check_qkv("k", k, kv_shape)
    _check_qkv("v", v, kv_shape)
    _check_qkv("o", o, shape)
    _check_lse(lse, shape)
    lib = _lib.load()
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    st = lib.fa_forward_offset(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                               int(kv_shape[2]), d, float(scale), int(bool(causal)), int(q_offset), kvp, sp)
    _lib.check(st, "fa_forward_offset")


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


def fa_backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len=None, stream=None):
    """C ``fa_backward_noalloc``: fa_backward_kvlen without a workspace (the library's own
    scratch array holds the row statistics); fills dq, dk, dv in place.  Problems whose
    statistics exceed NOALLOC_SCRATCH_BYTES raise FAError (FA_ERR_WORKSPACE)."""
    _check_qkv("q", q)
    shape = tuple(q.shape)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_qkv(name, t, shape)
    _check_lse(lse, shape)
    B, H, N, d = shape
    lib = _lib.load()
    kvp = _kv_ptr(kv_len, B, q.device)
    sp = _stream_ptr(stream, q.device)
    st = lib.fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                                 int(bool(causal)), kvp, sp)
    _lib.check(st, "fa_backward_noalloc")


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


# ---- FP8 forward ---------------------------------------------------------------------
FP8_BLOCK = 64  # rows per Q/K scale block, keys per V^T tile


def _check_dev(name, t, dtype, shape):
    torch = _torch()
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def fa_fp8_quantize_qk(x, x8, scales, signs=None, post_scale=1.0, stream=None):
    """C ``fa_fp8_quantize_qk``: fills x8 (E4M3 codes, uint8) and the 64-row block scales."""
    torch = _torch()
    _check_qkv("x", x)
    B, H, N, d = x.shape
    _check_dev("x8", x8, torch.uint8, (B, H, N, d))
    _check_dev("scales", scales, torch.float32, (B, H, -(-N // FP8_BLOCK)))
    sp_ = None
    if signs is not None:
        _check_dev("signs", signs, torch.float32, (d,))
        sp_ = signs.data_ptr()
    st = _lib.load().fa_fp8_quantize_qk(x.data_ptr(), x8.data_ptr(), scales.data_ptr(), sp_, float(post_scale),
                                        B, H, N, d, _stream_ptr(stream, x.device))
    _lib.check(st, "fa_fp8_quantize_qk")


def fa_fp8_quantize_v(v, v8t, scales, stream=None):
    """C ``fa_fp8_quantize_v``: fills v8t (transposed E4M3 tiles) and the column scales."""
    torch = _torch()
    _check_qkv("v", v)
    B, H, N, d = v.shape
    _check_dev("v8t", v8t, torch.uint8, (B, H, -(-N // FP8_BLOCK), d, FP8_BLOCK))
    _check_dev("scales", scales, torch.float32, (B, H, d))
    st = _lib.load().fa_fp8_quantize_v(v.data_ptr(), v8t.data_ptr(), scales.data_ptr(), B, H, N, d,
                                       _stream_ptr(stream, v.device))
    _lib.check(st, "fa_fp8_quantize_v")


def fa_forward_fp8(q8, sq, k8, sk, v8t, sv, o, lse, scale, causal, kv_len=None, stream=None):
    """C ``fa_forward_fp8``: fills o (bf16) and lse (fp32) in place."""
    torch = _torch()
    _check_qkv("o", o)
    B, H, N, d = o.shape
    nb = -(-N // FP8_BLOCK)
    for name, t in (("q8", q8), ("k8", k8)):
        _check_dev(name, t, torch.uint8, (B, H, N, d))
    _check_dev("v8t", v8t, torch.uint8, (B, H, nb, d, FP8_BLOCK))
    for name, t in (("q_scale", sq), ("k_scale", sk)):
        _check_dev(name, t, torch.float32, (B, H, nb))
    _check_dev("v_scale", sv, torch.float32, (B, H, d))
    _check_lse(lse, (B, H, N, d))
    st = _lib.load().fa_forward_fp8(q8.data_ptr(), sq.data_ptr(), k8.data_ptr(), sk.data_ptr(), v8t.data_ptr(),
                                    sv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, float(scale),
                                    int(bool(causal)), _kv_ptr(kv_len, B, o.device), _stream_ptr(stream, o.device))
    _lib.check(st, "fa_forward_fp8")


def fp8_v8t_to_rows(v8t, N):
    """Codes of ``fa_fp8_quantize_v`` in natural [B, H, N, d] order (index bookkeeping of
    the documented layout only): byte 32*g + p of row c of tile t is V[64 t + key(g, p)][c]
    with key(g, p) = 32*(p//16) + 8*((p%16)//4) + 4*g + p%4."""
    torch = _torch()
    B, H, nb, d, _ = v8t.shape
    pos = torch.arange(FP8_BLOCK)
    g, p = pos // 32, pos % 32
    key = 32 * (p // 16) + 8 * ((p % 16) // 4) + 4 * g + p % 4
    inv = torch.empty_like(key)
    inv[key] = pos
    rows = v8t.permute(0, 1, 2, 4, 3)[:, :, :, inv.to(v8t.device), :]  # [B, H, nb, 64 keys, d]
    return rows.reshape(B, H, nb * FP8_BLOCK, d)[:, :, :N].contiguous()


def forward_fp8(q, k, v, causal=False, scale=None, kv_len=None, signs=None):
    """Quantise q, k, v (bf16) and run the FP8 forward; signs (fp32 [d] of +-1 on the GPU)
    turns on incoherent processing.  Returns (o, lse)."""
    torch = _torch()
    _check_qkv("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_qkv(name, t, q.shape)
    nb = -(-N // FP8_BLOCK)
    dev = q.device
    q8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    v8t = torch.empty((B, H, nb, d, FP8_BLOCK), dtype=torch.uint8, device=dev)
    sq = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    sk = torch.empty_like(sq)
    sv = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    fa_fp8_quantize_qk(q, q8, sq, signs, 1.0 / d if signs is not None else 1.0)
    fa_fp8_quantize_qk(k, k8, sk, signs, 1.0)
    fa_fp8_quantize_v(v, v8t, sv)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    fa_forward_fp8(q8, sq, k8, sk, v8t, sv, o, lse, _default_scale(d, scale), causal, kv_len=kv_len)
    return o, lse
