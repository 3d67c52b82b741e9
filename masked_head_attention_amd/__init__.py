"""masked_head_attention_amd: fused masked multi-head attention forward for
AMD Instinct MI355X (gfx950).

Thin binding over libmha's C ABI (include/mha.h): it checks each tensor's
device, dtype, shape and contiguity, allocates the output if asked, and passes
raw device pointers plus the current HIP stream. Every step of the attention
runs in the HIP kernels of libmha; nothing here computes.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from ._abi import (ADDITIVE, BF16, CAUSAL, F16, F32, FLAG_BAD_LENGTH, FLAG_FULLY_MASKED_ROW,
                   FLAG_NONFINITE, KEEP, MASK_NONE, PADDING, PER_HEAD, MhaError, check, lib)

__all__ = ["fwd", "prenorm_cross_fwd", "softmax_rows", "decode", "decode_workspace_size",
           "bwd", "bwd_workspace_size",
           "get_flags", "set_debug_counters",
           "tile_config", "init", "MhaError", "CAUSAL", "PADDING", "ADDITIVE", "KEEP", "PER_HEAD",
           "MASK_NONE",
           "FLAG_FULLY_MASKED_ROW", "FLAG_NONFINITE", "FLAG_BAD_LENGTH"]


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return codes[t.dtype]


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _mask_arg(mask, kind, B, H, Lq, Lk, dtype):
    """Lengths [B] (PADDING), or a mask tensor (ADDITIVE, KEEP) [B,1,Lq,Lk], or
    [B,H,Lq,Lk] with PER_HEAD."""
    torch = _torch()
    if kind & PADDING:
        return _dev(mask, "mask (lengths)", torch.int32, (B,))
    if kind & (ADDITIVE | KEEP):
        return _dev(mask, "mask (tensor)", dtype, (B, H if kind & PER_HEAD else 1, Lq, Lk))
    if mask is not None:
        raise ValueError("mask given but mask kind has no PADDING, ADDITIVE or KEEP")
    return None


def init() -> None:
    """Allocate the current device's flag word (optional; see mha_init)."""
    check(lib().mha_init(), "mha_init")


def fwd(q, k, v, mask=None, kind: int = MASK_NONE, scale: Optional[float] = None, out=None,
        stream=None):
    """Masked MHA forward. q [B,H,Lq,D], k/v [B,H,Lk,D] -> out [B,H,Lq,D]."""
    torch = _torch()
    _dev(q, "q")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    _dev(k, "k", q.dtype, (B, H, Lk, D))
    _dev(v, "v", q.dtype, (B, H, Lk, D))
    m = _mask_arg(mask, kind, B, H, Lq, Lk, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, (B, H, Lq, D))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib().mha_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(m), kind, B, H, Lq, Lk, D, scale,
                       _dtype_code(q), _stream(stream), _ptr(out))
    check(st, "mha_fwd")
    return out


def prenorm_cross_workspace_size(B: int, H: int, Lq: int, Lk: int, D: int, dtype: int) -> int:
    """Bytes of workspace prenorm_cross_fwd(..., workspace=...) needs (0 unless bfloat16)."""
    n = ctypes.c_size_t(0)
    check(lib().mha_prenorm_cross_workspace_size(B, H, Lq, Lk, D, dtype, ctypes.byref(n)),
          "mha_prenorm_cross_workspace_size")
    return int(n.value)


def prenorm_cross_fwd(x, k, v, gamma, beta, eps: float = 1e-5, residual=None, mask=None,
                      kind: int = MASK_NONE, scale: Optional[float] = None, out=None, stream=None,
                      workspace=None):
    """Pre-LN cross-attention + residual. x [B,Lq,H*D], k/v [B,H,Lk,D] -> out [B,Lq,H*D].
    ``workspace`` (a uint8 GPU tensor of prenorm_cross_workspace_size(...) bytes)
    selects mha_prenorm_cross_fwd_ws: bfloat16 K and V are copied to float16,
    and the tokens' LayerNorm statistics computed, once per call instead of
    inside every attention workgroup."""
    torch = _torch()
    _dev(x, "x")
    B, Lq, F = x.shape
    _, H, Lk, D = k.shape
    if H * D != F:
        raise ValueError("x feature width must equal H*D")
    _dev(k, "k", x.dtype, (B, H, Lk, D))
    _dev(v, "v", x.dtype, (B, H, Lk, D))
    _dev(gamma, "gamma", x.dtype, (F,))
    _dev(beta, "beta", x.dtype, (F,))
    _dev(residual, "residual", x.dtype, (B, Lq, F))
    m = _mask_arg(mask, kind, B, H, Lq, Lk, x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (B, Lq, F))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None:
        st = lib().mha_prenorm_cross_fwd(_ptr(x), _ptr(k), _ptr(v), _ptr(m), kind, _ptr(gamma),
                                         _ptr(beta), float(eps), _ptr(residual), B, H, Lq, Lk, D,
                                         scale, _dtype_code(x), _stream(stream), _ptr(out))
        check(st, "mha_prenorm_cross_fwd")
        return out
    _dev(workspace, "workspace", torch.uint8)
    st = lib().mha_prenorm_cross_fwd_ws(_ptr(x), _ptr(k), _ptr(v), _ptr(m), kind, _ptr(gamma),
                                        _ptr(beta), float(eps), _ptr(residual), B, H, Lq, Lk, D,
                                        scale, _dtype_code(x), _ptr(workspace), workspace.numel(),
                                        _stream(stream), _ptr(out))
    check(st, "mha_prenorm_cross_fwd_ws")
    return out


def softmax_rows(s, out=None, scale: float = 1.0, stream=None):
    """Row softmax over the last axis of a materialised score tensor:
    out[..., j] = exp(scale*s[..., j] - max) / sum exp(scale*s - max); -inf
    entries get weight 0. out may be s itself (in place)."""
    torch = _torch()
    _dev(s, "s")
    cols = s.shape[-1] if s.dim() else 1
    rows = s.numel() // cols if cols else 0
    if out is None:
        out = torch.empty_like(s)
    _dev(out, "out", s.dtype, tuple(s.shape))
    st = lib().mha_softmax_rows(_ptr(s), _ptr(out), rows, cols, float(scale), _dtype_code(s),
                                _stream(stream))
    check(st, "mha_softmax_rows")
    return out


def decode_workspace_size(B: int, H: int, Lk: int, D: int, dtype_code: int) -> int:
    """Bytes of device workspace that decode needs for these sizes (0 if none)."""
    n = ctypes.c_size_t(0)
    check(lib().mha_decode_workspace_size(B, H, Lk, D, dtype_code, ctypes.byref(n)),
          "mha_decode_workspace_size")
    return int(n.value)


def decode(q, k, v, lens=None, scale: Optional[float] = None, out=None, lse=None,
           with_lse: bool = True, workspace=None, stream=None):
    """One new query row per (b, h) against a key/value cache.
    q [B,H,D], k/v [B,H,Lk,D], lens int32 [B] or None -> (out [B,H,D], lse
    float32 [B,H] or None). ``workspace`` is a uint8 GPU tensor of at least
    decode_workspace_size(...) bytes; when omitted one is allocated here."""
    torch = _torch()
    _dev(q, "q")
    B, H, D = q.shape
    Lk = k.shape[2]
    _dev(k, "k", q.dtype, (B, H, Lk, D))
    _dev(v, "v", q.dtype, (B, H, Lk, D))
    _dev(lens, "lens", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, (B, H, D))
    if lse is None and with_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _dev(lse, "lse", torch.float32, (B, H))
    code = _dtype_code(q)
    need = decode_workspace_size(B, H, Lk, D, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib().mha_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(lens), B, H, Lk, D, scale, code,
                              _ptr(workspace), ws_bytes, _stream(stream), _ptr(out), _ptr(lse))
    check(st, "mha_decode_fwd")
    return out, lse


def noalloc_scratch_bytes() -> int:
    """Size of the per-GPU static scratch array of the allocation-free entry points."""
    n = ctypes.c_size_t(0)
    check(lib().mha_noalloc_scratch_bytes(ctypes.byref(n)), "mha_noalloc_scratch_bytes")
    return int(n.value)


def decode_noalloc(q, k, v, lens=None, scale: Optional[float] = None, out=None, lse=None,
                   stream=None):
    """decode() through the allocation-free entry point: the library allocates
    nothing and takes no workspace (the partial results live in its static
    per-GPU scratch array). init() must have run on the device. ``out`` and
    ``lse`` must be given (the caller's buffers); lse may be None."""
    _dev(q, "q")
    B, H, D = q.shape
    Lk = k.shape[2]
    _dev(k, "k", q.dtype, (B, H, Lk, D))
    _dev(v, "v", q.dtype, (B, H, Lk, D))
    _dev(lens, "lens", _torch().int32, (B,))
    if out is None:
        raise ValueError("decode_noalloc: out must be given (this entry point allocates nothing)")
    _dev(out, "out", q.dtype, (B, H, D))
    _dev(lse, "lse", _torch().float32, (B, H))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib().mha_decode_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(lens), B, H, Lk, D, scale,
                                      _dtype_code(q), _stream(stream), _ptr(out), _ptr(lse))
    check(st, "mha_decode_fwd_noalloc")
    return out, lse


def bwd_workspace_size(B: int, H: int, Lq: int, dtype_code: int) -> int:
    """Bytes of device workspace that bwd needs (the rows' statistics)."""
    n = ctypes.c_size_t(0)
    check(lib().mha_bwd_workspace_size(B, H, Lq, dtype_code, ctypes.byref(n)),
          "mha_bwd_workspace_size")
    return int(n.value)


def bwd(q, k, v, dout, mask=None, kind: int = MASK_NONE, scale: Optional[float] = None,
        dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of fwd for the upstream gradient dout: q, dout [B,H,Lq,D],
    k, v [B,H,Lk,D] -> (dq, dk, dv). ``workspace`` is a uint8 GPU tensor of at least
    bwd_workspace_size(...) bytes; when omitted one is allocated here."""
    torch = _torch()
    _dev(q, "q")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    _dev(k, "k", q.dtype, (B, H, Lk, D))
    _dev(v, "v", q.dtype, (B, H, Lk, D))
    _dev(dout, "dout", q.dtype, (B, H, Lq, D))
    m = _mask_arg(mask, kind, B, H, Lq, Lk, q.dtype)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _dev(dq, "dq", q.dtype, (B, H, Lq, D))
    _dev(dk, "dk", q.dtype, (B, H, Lk, D))
    _dev(dv, "dv", q.dtype, (B, H, Lk, D))
    code = _dtype_code(q)
    need = bwd_workspace_size(B, H, Lq, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib().mha_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(m), kind, B, H, Lq, Lk, D,
                       scale, code, _ptr(workspace), ws_bytes, _stream(stream), _ptr(dq), _ptr(dk),
                       _ptr(dv))
    check(st, "mha_bwd")
    return dq, dk, dv


def get_flags(clear: bool = True, stream=None) -> int:
    """Synchronise the stream and read (and by default clear) the device flag word."""
    f = ctypes.c_uint32(0)
    check(lib().mha_get_flags(_stream(stream), ctypes.byref(f), int(clear)), "mha_get_flags")
    return int(f.value)


def set_debug_counters(counters) -> None:
    """Point the kernels at an int64 GPU tensor of 3 counters, or None to stop."""
    torch = _torch()
    if counters is not None:
        _dev(counters, "counters", torch.int64, (3,))
    check(lib().mha_set_debug_counters(_ptr(counters)), "mha_set_debug_counters")


def tile_config(dtype_code: int, D: int, kind: int = MASK_NONE):
    """(rows, keys) of the tile the skip decision is made on."""
    r, k = ctypes.c_int(0), ctypes.c_int(0)
    check(lib().mha_tile_config(dtype_code, D, kind, ctypes.byref(r), ctypes.byref(k)),
          "mha_tile_config")
    return r.value, k.value
