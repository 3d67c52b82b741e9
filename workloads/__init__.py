"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests, the benchmark and the smoke check; it feeds both the GPU
library and the fp64 oracle. It holds none of the attention arithmetic: it
draws numbers, rounds them to the storage dtype and packs masks.

Recipe (fixed, so a seed names one input exactly):
  * numpy ``default_rng(seed)`` (PCG64); values are drawn in float64;
  * draw order: q, k, v, then padding lengths, then the block pattern, then x,
    gamma, beta (a tensor a workload does not have is not drawn);
  * rounding to the storage dtype: float32 by ``astype``; float16 by ``astype``
    (round to nearest even); bfloat16 by rounding the float32 value to nearest
    even on its upper 16 bits (numpy has no bfloat16, so bf16 tensors travel as
    uint16 bit patterns);
  * the float64 copies handed to the oracle are the rounded values, widened
    exactly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CAUSAL, PADDING, ADDITIVE, KEEP, PER_HEAD = 1, 2, 4, 8, 16
DTYPES = ("f32", "f16", "bf16")


def _bf16_bits_from_f32(f32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    nan = np.isnan(f32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage representation of ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float16)
    if dtype == "bf16":
        return _bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


def to_f64(stored: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact float64 widening of a stored tensor."""
    if stored is None:
        return None
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored).astype(np.float64)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    kind: int
    B: int
    H: int
    Lq: int
    Lk: int
    D: int
    scale: float
    seed: int
    q: Optional[np.ndarray] = None  # [B,H,Lq,D] stored (absent for pre-LN)
    k: Optional[np.ndarray] = None  # [B,H,Lk,D]
    v: Optional[np.ndarray] = None  # [B,H,Lk,D]
    lens: Optional[np.ndarray] = None  # int32 [B] (PADDING)
    add: Optional[np.ndarray] = None  # [B,1,Lq,Lk] ([B,H,Lq,Lk] PER_HEAD) stored (ADDITIVE, KEEP)
    prenorm: bool = False
    x: Optional[np.ndarray] = None  # [B,Lq,H*D] stored (pre-LN)
    gamma: Optional[np.ndarray] = None  # [H*D]
    beta: Optional[np.ndarray] = None  # [H*D]
    eps: float = 1e-5
    residual: bool = False  # pre-LN: residual = x

    def f64(self, name: str) -> Optional[np.ndarray]:
        return to_f64(getattr(self, name), self.dtype)


def _normal(rng, shape, std=1.0, mean=0.0):
    return rng.standard_normal(shape) * std + mean


def make(name: str, dtype: str, B: int, H: int, Lq: int, Lk: int, D: int, kind: int = 0,
         seed: int = 0, qkv_std: float = 1.0, lens_range=None, block_p: float = 0.0,
         block: int = 32, prenorm: bool = False, x_mean: float = 0.0, x_std: float = 1.0,
         eps: float = 1e-5, residual: bool = False, scale: Optional[float] = None) -> Workload:
    """Draw one workload. ``lens_range`` (lo, hi) is inclusive. With ADDITIVE the
    mask holds -inf for keys >= len_b (when lens_range is given) and for each
    (b, query block, key block) of ``block`` x ``block`` chosen with probability
    ``block_p``; diagonal blocks are never chosen; legal entries are 0. With
    PER_HEAD the mask is [B,H,Lq,Lk], its blocks drawn per head, and legal
    entries hold biases 0.5 * N(0, 1). KEEP draws the same pattern into a
    keep-mask: 0 where masked, U(0.5, 2) where legal."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    w = Workload(name=name, dtype=dtype, kind=kind, B=B, H=H, Lq=Lq, Lk=Lk, D=D,
                 scale=(1.0 / math.sqrt(D)) if scale is None else scale, seed=seed,
                 prenorm=prenorm, eps=eps, residual=residual)
    if not prenorm:
        w.q = round_to(_normal(rng, (B, H, Lq, D), qkv_std), dtype)
    w.k = round_to(_normal(rng, (B, H, Lk, D), qkv_std), dtype)
    w.v = round_to(_normal(rng, (B, H, Lk, D), qkv_std), dtype)
    lens = None
    if lens_range is not None:
        lens = rng.integers(lens_range[0], lens_range[1] + 1, size=B).astype(np.int32)
    if kind & PADDING:
        if lens is None:
            raise ValueError("PADDING needs lens_range")
        w.lens = lens
    if kind & (ADDITIVE | KEEP):
        Hm = H if kind & PER_HEAD else 1
        masked = np.zeros((B, Hm, Lq, Lk), bool)
        if lens is not None and not (kind & PADDING):
            for b in range(B):
                masked[b, :, :, lens[b]:] = True
        if block_p > 0.0:
            nqb, nkb = -(-Lq // block), -(-Lk // block)
            pick = rng.random((B, Hm, nqb, nkb)) < block_p
            for b, h, qb, kb in zip(*np.nonzero(pick)):
                if qb == kb:
                    continue
                masked[b, h, qb * block:(qb + 1) * block, kb * block:(kb + 1) * block] = True
        if kind & ADDITIVE:
            legal = _normal(rng, masked.shape, 0.5) if kind & PER_HEAD else 0.0
            add = np.where(masked, -np.inf, legal)
        else:
            add = np.where(masked, 0.0, rng.uniform(0.5, 2.0, masked.shape))
        w.add = round_to(add, dtype)
    if prenorm:
        F = H * D
        w.x = round_to(_normal(rng, (B, Lq, F), x_std, x_mean), dtype)
        w.gamma = round_to(rng.uniform(0.5, 1.5, F), dtype)
        w.beta = round_to(_normal(rng, (F,), 0.1), dtype)
    return w


# The five workloads named for this path, with their full sizes.
CONFIGS = {
    1: dict(name="tiny-causal-f32", dtype="f32", B=2, H=2, Lq=32, Lk=32, D=16, kind=CAUSAL,
            seed=1),
    2: dict(name="latency-causal-padding-f32", dtype="f32", B=4, H=8, Lq=128, Lk=128, D=64,
            kind=CAUSAL | PADDING, lens_range=(64, 128), seed=2),
    3: dict(name="llama2-7b-causal-f16", dtype="f16", B=1, H=32, Lq=2048, Lk=2048, D=128,
            kind=CAUSAL, qkv_std=0.5, seed=3),
    4: dict(name="prenorm-cross-bf16", dtype="bf16", B=32, H=16, Lq=2048, Lk=2048, D=64, kind=0,
            prenorm=True, x_mean=0.5, x_std=3.0, eps=1e-5, residual=True, seed=4),
    5: dict(name="varlen-additive-f16", dtype="f16", B=16, H=8, Lq=512, Lk=512, D=64,
            kind=ADDITIVE, lens_range=(64, 512), block_p=0.1, block=32, seed=5),
}


def config(n: int, **overrides) -> Workload:
    """Workload n at its full size, or with overridden sizes/seed (same recipe)."""
    spec = dict(CONFIGS[n])
    spec.update(overrides)
    return make(**spec)


# ---- the standalone row-softmax workload -----------------------------------
@dataclasses.dataclass
class ScoreRows:
    """A materialised score tensor whose last axis is one softmax row."""
    name: str
    dtype: str
    shape: tuple
    scale: float
    seed: int
    s: Optional[np.ndarray] = None  # stored scores, `shape`

    @property
    def rows(self) -> int:
        return int(np.prod(self.shape[:-1]))

    @property
    def cols(self) -> int:
        return int(self.shape[-1])

    def f64(self, name: str = "s") -> Optional[np.ndarray]:
        return to_f64(getattr(self, name), self.dtype)


def make_scores(name: str, dtype: str, shape, seed: int = 0, std: float = 2.0,
                masked_p: float = 0.0, masked_rows: int = 0, scale: float = 1.0) -> ScoreRows:
    """Scores ~ std * N(0, 1) rounded to ``dtype``; then, in this order, each
    entry is set to -inf with probability ``masked_p`` and the first
    ``masked_rows`` rows (in a random choice) entirely to -inf."""
    rng = np.random.default_rng(seed)
    shape = tuple(int(d) for d in shape)
    x = _normal(rng, shape, std)
    if masked_p > 0:
        x = np.where(rng.random(shape) < masked_p, -np.inf, x)
    if masked_rows > 0:
        flat = x.reshape(-1, shape[-1])
        pick = rng.choice(flat.shape[0], size=min(masked_rows, flat.shape[0]), replace=False)
        flat[pick] = -np.inf
    return ScoreRows(name=name, dtype=dtype, shape=shape, scale=scale, seed=seed,
                     s=round_to(x, dtype))


# the pages' row-softmax workload: a 1 x 32 x 2048 x 2048 float16 score tensor
SOFTMAX_CONFIG = dict(name="rows-softmax-f16", dtype="f16", shape=(1, 32, 2048, 2048), seed=6,
                      std=2.0)


def softmax_config(**overrides) -> ScoreRows:
    spec = dict(SOFTMAX_CONFIG)
    spec.update(overrides)
    return make_scores(**spec)


# ---- the decode workload -----------------------------------------------------
# One new token per sequence against a Llama-2-7B-shaped key/value cache
# (H=32, D=128, float16) of capacity 4096, per-sequence cache lengths uniform
# in [256, 4096]; q, k, v = 0.5 * N(0, 1) as in the causal Llama-2 workload.
# Drawn by `make` with Lq = 1 (q [B,H,1,D] is the decode layout [B,H,D]) and
# the padding lengths as the cache lengths.
DECODE_CONFIG = dict(name="llama2-7b-decode-f16", dtype="f16", B=16, H=32, Lq=1, Lk=4096, D=128,
                     kind=PADDING, lens_range=(256, 4096), qkv_std=0.5, seed=7)


def decode_config(**overrides) -> Workload:
    spec = dict(DECODE_CONFIG)
    spec.update(overrides)
    if spec.get("Lq", 1) != 1:
        raise ValueError("decode has one query row")
    return make(**spec)


# ---- the upstream gradient of the backward -------------------------------------
def grad_output(w: Workload, std: float = 1.0) -> np.ndarray:
    """dO for workload w: std * N(0, 1) of the output's shape [B,H,Lq,D], rounded
    to the workload's dtype, drawn from its own stream default_rng(seed + 7919)
    so the workload's other tensors are unchanged."""
    rng = np.random.default_rng(w.seed + 7919)
    return round_to(_normal(rng, (w.B, w.H, w.Lq, w.D), std), w.dtype)


# The backward workload: the gradients of the causal Llama-2-7B-shaped
# self-attention (workload 3's shapes and draws), dO ~ N(0, 1).
BWD_CONFIG = 3
