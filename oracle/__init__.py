"""Plain fp64 CPU reference for the masked multi-head attention forward (and
its backward, decode and row-softmax variants).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark are the only callers. The GPU library never
imports, links or runs anything here, and nothing here imports the GPU package.

The arithmetic lives in ``mha_oracle.c`` (built into ``liboracle.so`` by
``oracle/build.py``); this module only marshals numpy arrays into it. Every
array handed in is float64 (inputs are the same dtype-rounded values the GPU
receives, widened exactly), int32 for padding lengths.

Parity status: every function here is pinned by tests that do not reuse its
code (brute force in exact decimal arithmetic, library special cases, closed
forms and invariants) -- none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

CAUSAL, PADDING, ADDITIVE, KEEP, PER_HEAD = 1, 2, 4, 8, 16
TENSOR = ADDITIVE | KEEP  # kinds that read a mask tensor
FLAG_FULLY_MASKED_ROW, FLAG_NONFINITE, FLAG_BAD_LENGTH = 1, 2, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)
_bp = ctypes.POINTER(ctypes.c_uint8)
_i, _u, _d, _l = ctypes.c_int, ctypes.c_uint, ctypes.c_double, ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_threads": ([], _i),
        "oracle_set_threads": ([_i], None),
        "oracle_mha_fwd": ([_dp, _dp, _dp, _ip, _dp, _u, _i, _i, _i, _i, _i, _d, _dp], ctypes.c_uint32),
        "oracle_mha_rows": ([_dp, _dp, _dp, _ip, _dp, _u, _i, _i, _i, _i, _i, _d, _lp, _l, _dp],
                            ctypes.c_uint32),
        "oracle_probs_row": ([_dp, _dp, _ip, _dp, _u, _i, _i, _i, _i, _i, _d, _i, _i, _i, _dp],
                             ctypes.c_uint32),
        "oracle_layernorm": ([_dp, _dp, _dp, _d, _l, _i, _dp], None),
        "oracle_prenorm_rows": ([_dp, _dp, _dp, _ip, _dp, _u, _dp, _dp, _d, _dp, _i, _i, _i,
                                 _i, _i, _d, _lp, _l, _dp], ctypes.c_uint32),
        "oracle_prenorm_cross_fwd": ([_dp, _dp, _dp, _ip, _dp, _u, _dp, _dp, _d, _dp, _i, _i,
                                      _i, _i, _i, _d, _dp], ctypes.c_uint32),
        "oracle_mask_decisions": ([_ip, _dp, _u, _i, _i, _i, _i, _bp], None),
        "oracle_softmax_rows": ([_dp, _l, _i, _d, _dp], ctypes.c_uint32),
        "oracle_decode": ([_dp, _dp, _dp, _ip, _i, _i, _i, _i, _d, _dp, _dp], ctypes.c_uint32),
        "oracle_mha_bwd": ([_dp, _dp, _dp, _dp, _ip, _dp, _u, _i, _i, _i, _i, _i, _d, _dp, _dp,
                            _dp], ctypes.c_uint32),
        "oracle_unmasked_pairs": ([_ip, _dp, _u, _i, _i, _i, _i], _l),
        "oracle_tile_counts": ([_ip, _dp, _u, _i, _i, _i, _i, _i, _i, _lp], None),
        "oracle_fully_masked_rows": ([_ip, _dp, _u, _i, _i, _i, _i], _l),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _mask_args(kind, lens, add, B, Lq, Lk, H=1):
    """Padding lengths [B]; the mask tensor (additive or keep) [B,1,Lq,Lk], or
    [B,H,Lq,Lk] with PER_HEAD."""
    if kind & PADDING:
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("lens must have shape [B]")
    else:
        lens = None
    if kind & TENSOR:
        add = _f64(add, (B, H if kind & PER_HEAD else 1, Lq, Lk))
    else:
        add = None
    return lens, add


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def mha_fwd(q, k, v, kind=0, lens=None, add=None, scale=None):
    """Full forward. q [B,H,Lq,D], k/v [B,H,Lk,D] -> (out [B,H,Lq,D], flags)."""
    q = _f64(q)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    k = _f64(k, (B, H, Lk, D))
    v = _f64(v, (B, H, Lk, D))
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((B, H, Lq, D), np.float64)
    f = _load().oracle_mha_fwd(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(lens, _ip),
                               _ptr(add, _dp), kind, B, H, Lq, Lk, D, scale, _ptr(out, _dp))
    return out, int(f)


def mha_rows(q, k, v, rows, kind=0, lens=None, add=None, scale=None):
    """Selected rows; rows is an int array [n,3] of (b, h, i). -> (out [n,D], flags)."""
    q = _f64(q)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    k = _f64(k, (B, H, Lk, D))
    v = _f64(v, (B, H, Lk, D))
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    f = _load().oracle_mha_rows(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(lens, _ip),
                                _ptr(add, _dp), kind, B, H, Lq, Lk, D, scale,
                                _ptr(rows, _lp), rows.shape[0], _ptr(out, _dp))
    return out, int(f)


def probs_row(q, k, b, h, i, kind=0, lens=None, add=None, scale=None):
    """Softmax weights of one row -> (p [Lk], flags)."""
    q = _f64(q)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    k = _f64(k, (B, H, Lk, D))
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    p = np.empty(Lk, np.float64)
    f = _load().oracle_probs_row(_ptr(q, _dp), _ptr(k, _dp), _ptr(lens, _ip), _ptr(add, _dp),
                                 kind, B, H, Lq, Lk, D, scale, b, h, i, _ptr(p, _dp))
    return p, int(f)


def layernorm(x, gamma, beta, eps):
    """Per-token LayerNorm over the last axis of x, in fp64."""
    x = _f64(x)
    F = x.shape[-1]
    gamma = _f64(gamma, (F,))
    beta = _f64(beta, (F,))
    y = np.empty_like(x)
    _load().oracle_layernorm(_ptr(x, _dp), _ptr(gamma, _dp), _ptr(beta, _dp), float(eps),
                             x.size // F, F, _ptr(y, _dp))
    return y


def _prenorm_common(x, k, v, gamma, beta, residual, kind, lens, add, scale):
    x = _f64(x)
    B, Lq, F = x.shape
    _, H, Lk, D = k.shape
    if H * D != F:
        raise ValueError("x feature width must equal H*D")
    k = _f64(k, (B, H, Lk, D))
    v = _f64(v, (B, H, Lk, D))
    gamma = _f64(gamma, (F,))
    beta = _f64(beta, (F,))
    residual = _f64(residual, (B, Lq, F)) if residual is not None else None
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    return x, k, v, gamma, beta, residual, lens, add, scale, (B, H, Lq, Lk, D)


def prenorm_cross_fwd(x, k, v, gamma, beta, eps, residual=None, kind=0, lens=None, add=None,
                      scale=None):
    """Full pre-LN cross-attention. x [B,Lq,H*D] -> (out [B,Lq,H*D], flags).
    The normalised query is used in fp64 as computed (no rounding step)."""
    x, k, v, gamma, beta, residual, lens, add, scale, (B, H, Lq, Lk, D) = _prenorm_common(
        x, k, v, gamma, beta, residual, kind, lens, add, scale)
    out = np.empty((B, Lq, H * D), np.float64)
    f = _load().oracle_prenorm_cross_fwd(
        _ptr(x, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(lens, _ip), _ptr(add, _dp), kind,
        _ptr(gamma, _dp), _ptr(beta, _dp), float(eps), _ptr(residual, _dp), B, H, Lq,
        Lk, D, scale, _ptr(out, _dp))
    return out, int(f)


def prenorm_rows(x, k, v, gamma, beta, eps, rows, residual=None, kind=0, lens=None, add=None,
                 scale=None):
    """Selected rows (b, i, h) of the pre-LN cross-attention -> (out [n,D], flags)."""
    x, k, v, gamma, beta, residual, lens, add, scale, (B, H, Lq, Lk, D) = _prenorm_common(
        x, k, v, gamma, beta, residual, kind, lens, add, scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    f = _load().oracle_prenorm_rows(
        _ptr(x, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(lens, _ip), _ptr(add, _dp), kind,
        _ptr(gamma, _dp), _ptr(beta, _dp), float(eps), _ptr(residual, _dp), B, H,
        Lq, Lk, D, scale, _ptr(rows, _lp), rows.shape[0], _ptr(out, _dp))
    return out, int(f)


def mask_decisions(kind, B, Lq, Lk, lens=None, add=None, H=1):
    """uint8 [B,Lq,Lk], 1 where the pair is masked; [B,H,Lq,Lk] with PER_HEAD."""
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    Hm = H if kind & PER_HEAD else 1
    dec = np.empty((B, Hm, Lq, Lk), np.uint8)
    _load().oracle_mask_decisions(_ptr(lens, _ip), _ptr(add, _dp), kind, B, H, Lq, Lk,
                                  _ptr(dec, _bp))
    return dec if kind & PER_HEAD else dec[:, 0]


def unmasked_pairs(kind, B, H, Lq, Lk, lens=None, add=None) -> int:
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    return int(_load().oracle_unmasked_pairs(_ptr(lens, _ip), _ptr(add, _dp), kind, B, H, Lq, Lk))


def tile_counts(kind, B, H, Lq, Lk, rm, bn, lens=None, add=None):
    """(computed, skipped) tiles of rm rows x bn keys, summed over b and h."""
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    c = np.zeros(2, np.int64)
    _load().oracle_tile_counts(_ptr(lens, _ip), _ptr(add, _dp), kind, B, H, Lq, Lk, rm, bn,
                               _ptr(c, _lp))
    return int(c[0]), int(c[1])


def fully_masked_rows(kind, B, H, Lq, Lk, lens=None, add=None) -> int:
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    return int(_load().oracle_fully_masked_rows(_ptr(lens, _ip), _ptr(add, _dp), kind, B, H,
                                                Lq, Lk))


def softmax_rows(s, scale=1.0):
    """Row softmax of a materialised score array (last axis = one row):
    p = exp(scale*s - max) / sum exp(scale*s - max), three passes per row
    ["Why attention must compute the max first" 2.1]. Entries equal to -inf are
    masked (weight 0); a row with every entry masked gives zeros and
    FLAG_FULLY_MASKED_ROW. Returns (p, flags)."""
    s = _f64(s)
    cols = s.shape[-1] if s.ndim else 1
    rows = s.size // cols if cols else 0
    p = np.zeros(s.shape, np.float64)
    f = _load().oracle_softmax_rows(_ptr(s, _dp), rows, cols, float(scale), _ptr(p, _dp))
    return p, int(f)


def decode(q, k, v, lens=None, scale=None):
    """One query row per (b, h): q [B,H,D], k/v [B,H,Lk,D], optional key
    lengths [B]. Returns (out [B,H,D], lse [B,H], flags); lse is the natural
    log-sum-exp of the legal scaled scores (-inf for a row with none)."""
    q = _f64(q)
    B, H, D = q.shape
    Lk = k.shape[2]
    k = _f64(k, (B, H, Lk, D))
    v = _f64(v, (B, H, Lk, D))
    if lens is not None:
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("lens must have shape [B]")
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((B, H, D), np.float64)
    lse = np.empty((B, H), np.float64)
    f = _load().oracle_decode(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(lens, _ip), B, H, Lk,
                              D, scale, _ptr(out, _dp), _ptr(lse, _dp))
    return out, lse, int(f)


def mha_bwd(q, k, v, dout, kind=0, lens=None, add=None, scale=None):
    """Gradients of mha_fwd for the upstream gradient dout [B,H,Lq,D]
    ("Why attention must compute the max first" 3.3: the softmax Jacobian).
    Returns (dq [B,H,Lq,D], dk, dv [B,H,Lk,D], flags)."""
    q = _f64(q)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    k = _f64(k, (B, H, Lk, D))
    v = _f64(v, (B, H, Lk, D))
    dout = _f64(dout, (B, H, Lq, D))
    lens, add = _mask_args(kind, lens, add, B, Lq, Lk, H)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    f = _load().oracle_mha_bwd(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(dout, _dp),
                               _ptr(lens, _ip), _ptr(add, _dp), int(kind), B, H, Lq, Lk, D, scale,
                               _ptr(dq, _dp), _ptr(dk, _dp), _ptr(dv, _dp))
    return dq, dk, dv, int(f)
