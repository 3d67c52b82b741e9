"""Shared test helpers: moving seeded workloads to the GPU, running both sides,
and the parity bar |gpu - oracle| <= tol + half an output ulp."""
from __future__ import annotations

import math

import numpy as np

import oracle
import workloads as W

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
MANT = {"f32": 23, "f16": 10, "bf16": 7}
EMIN = {"f32": -126, "f16": -14, "bf16": -126}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output dtype at |x| (the rounding
    of the stored output that no kernel can avoid)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, EMIN[dtype])
    return 0.5 * np.exp2(e - MANT[dtype])


def parity_error(gpu: np.ndarray, ref: np.ndarray, dtype: str):
    """(max |err|, max of |err| / allowed) over all elements."""
    err = np.abs(gpu - ref)
    allowed = TOL[dtype] + half_ulp(ref, dtype)
    return float(err.max(initial=0.0)), float((err / allowed).max(initial=0.0))


def assert_parity(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all() == np.isfinite(ref).all(), what
    err, ratio = parity_error(gpu, ref, dtype)
    if ratio > 1.0:
        idx = np.unravel_index(np.argmax(np.abs(gpu - ref) / (TOL[dtype] + half_ulp(ref, dtype))),
                               gpu.shape)
        raise AssertionError(f"{what}: parity failed, max err {err:.3e}, worst at {idx}: "
                             f"gpu {gpu[idx]!r} oracle {ref[idx]!r} (ratio {ratio:.2f})")
    return err


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(arr, dtype: str):
    import torch

    if arr is None:
        return None
    if arr.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def from_dev(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_inputs(w: W.Workload):
    d = {}
    for name in ("q", "k", "v", "x", "gamma", "beta"):
        d[name] = to_dev(getattr(w, name), w.dtype)
    if w.kind & W.PADDING:
        d["mask"] = to_dev(w.lens, w.dtype)
    elif w.kind & (W.ADDITIVE | W.KEEP):
        d["mask"] = to_dev(w.add, w.dtype)
    else:
        d["mask"] = None
    return d


def prenorm_workspace(w: W.Workload):
    """A workspace of the size mha_prenorm_cross_fwd_ws asks for, filled with a
    byte pattern (its contents need no initialisation)."""
    import torch

    import masked_head_attention_amd as M

    code = {"f32": M.F32, "f16": M.F16, "bf16": M.BF16}[w.dtype]
    need = M.prenorm_cross_workspace_size(w.B, w.H, w.Lq, w.Lk, w.D, code)
    return torch.full((max(need, 1),), 0x5A, dtype=torch.uint8, device="cuda")


def run_gpu(w: W.Workload, inputs=None, out=None, workspace=None):
    """One call of the library on workload w; returns (out tensor, flags).
    A pre-LN call with ``workspace`` goes through mha_prenorm_cross_fwd_ws."""
    import masked_head_attention_amd as M

    d = inputs if inputs is not None else gpu_inputs(w)
    M.get_flags(clear=True)
    if w.prenorm:
        o = M.prenorm_cross_fwd(d["x"], d["k"], d["v"], d["gamma"], d["beta"], w.eps,
                                residual=d["x"] if w.residual else None, mask=d["mask"],
                                kind=w.kind, scale=w.scale, out=out, workspace=workspace)
    else:
        o = M.fwd(d["q"], d["k"], d["v"], mask=d["mask"], kind=w.kind, scale=w.scale, out=out)
    return o, M.get_flags(clear=True)


def run_oracle(w: W.Workload):
    if w.prenorm:
        x = w.f64("x")
        return oracle.prenorm_cross_fwd(x, w.f64("k"), w.f64("v"), w.f64("gamma"),
                                        w.f64("beta"), w.eps, residual=x if w.residual else None,
                                        kind=w.kind, lens=w.lens, add=w.f64("add"),
                                        scale=w.scale)
    return oracle.mha_fwd(w.f64("q"), w.f64("k"), w.f64("v"), w.kind, w.lens, w.f64("add"),
                          w.scale)
