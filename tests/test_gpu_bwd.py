"""GPU parity of the backward (the gradients dQ, dK, dV of the masked
attention forward for an upstream gradient dO, through the softmax Jacobian of
"Why attention must compute the max first", section 3.3) against the fp64
oracle, through the C ABI.

Bar: |gpu - oracle| <= 2e-3 (float16 / bfloat16) or 1e-5 (float32) + half an
output ulp elementwise for every gradient; flags agree exactly.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import assert_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_head_attention_amd as M

    M.init()
    M.get_flags(clear=True)
    yield


def _run(w, g):
    import masked_head_attention_amd as M

    print(f"[bwd] {w.name} {w.dtype} B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} D{w.D} kind {w.kind} "
          f"seed {w.seed}", flush=True)
    q, k, v = (to_dev(getattr(w, n), w.dtype) for n in ("q", "k", "v"))
    mask = (to_dev(w.lens, w.dtype) if w.kind & W.PADDING else
            to_dev(w.add, w.dtype) if w.kind & (W.ADDITIVE | W.KEEP) else None)
    M.get_flags(clear=True)
    dq, dk, dv = M.bwd(q, k, v, to_dev(g, w.dtype), mask=mask, kind=w.kind, scale=w.scale)
    flags = M.get_flags(clear=True)
    return from_dev(dq), from_dev(dk), from_dev(dv), flags


def _check(w, what, std=1.0):
    g = W.grad_output(w, std)
    gq, gk, gv, flags = _run(w, g)
    rq, rk, rv, rflags = oracle.mha_bwd(w.f64("q"), w.f64("k"), w.f64("v"), W.to_f64(g, w.dtype),
                                        w.kind, w.lens, w.f64("add"), w.scale)
    for name, a, b in [("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)]:
        assert_parity(a, b, w.dtype, f"{what} {name}")
    assert flags == rflags, (what, flags, rflags)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", [0, W.CAUSAL, W.PADDING, W.CAUSAL | W.PADDING])
def test_bwd_parity(dtype, D, kind):
    L = 100 if D == 128 else 130
    lr = (1, L) if kind & W.PADDING else None
    w = W.make(f"bwd-{dtype}-{D}", dtype, 2, 3, L, L, D, kind=kind, seed=D + kind,
               lens_range=lr)
    _check(w, f"bwd-{dtype}-D{D}-kind{kind}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kind", [W.ADDITIVE, W.ADDITIVE | W.CAUSAL, W.KEEP,
                                  W.ADDITIVE | W.PER_HEAD, W.KEEP | W.PER_HEAD | W.CAUSAL])
def test_bwd_tensor_masks(dtype, kind):
    """Additive and keep masks, shared or one slab per head, with -inf / 0
    blocks, key padding folded into the tensor and ragged sizes (Lk odd)."""
    w = W.make("bwd-masks", dtype, 2, 3, 77, 93, 64, kind=kind, seed=40 + kind,
               lens_range=(10, 93), block_p=0.25, block=16)
    _check(w, f"bwd-mask-{dtype}-{kind}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (33, 70), (70, 33), (64, 64), (5, 200)])
def test_bwd_shapes(dtype, Lq, Lk):
    w = W.make("bwd-shapes", dtype, 1, 2, Lq, Lk, 64, seed=Lq * 7 + Lk, qkv_std=1.5)
    _check(w, f"bwd-shape-{dtype}-{Lq}x{Lk}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_zero_lengths_and_flags(dtype):
    w = W.make("bwd-len0", dtype, 3, 2, 40, 40, 64, kind=W.PADDING | W.CAUSAL, seed=31,
               lens_range=(0, 40))
    w.lens = np.array([0, 40, 17], np.int32)
    _check(w, f"bwd-len0-{dtype}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_bwd_out_of_range_lengths(dtype):
    """Lengths below 0 or above Lk act clamped (no key; every key) and raise
    the bad-length flag, as in the forward; the clamped-to-0 rows are fully
    masked."""
    w = W.make("bwd-badlen", dtype, 3, 2, 40, 40, 64, kind=W.PADDING, seed=33,
               lens_range=(1, 40))
    w.lens = np.array([-3, 57, 17], np.int32)
    _check(w, f"bwd-badlen-{dtype}")


def test_bwd_large_gradients():
    w = W.make("bwd-large", "f16", 1, 4, 96, 96, 64, kind=W.CAUSAL, seed=32, qkv_std=2.0)
    _check(w, "bwd-large", std=4.0)


def test_bwd_workload_full_size():
    """The backward at the causal Llama-2-7B shape (the benchmark's workload),
    in the launch configuration the benchmark times: dq, dk and dv of every
    head against the oracle, four heads at a time."""
    w = W.config(W.BWD_CONFIG)
    g = W.grad_output(w)
    gq, gk, gv, flags = _run(w, g)
    assert flags == 0
    q, k, v, g64 = w.f64("q"), w.f64("k"), w.f64("v"), W.to_f64(g, w.dtype)
    for h0 in range(0, w.H, 4):
        sl = slice(h0, h0 + 4)
        rq, rk, rv, rflags = oracle.mha_bwd(q[:, sl], k[:, sl], v[:, sl], g64[:, sl], w.kind,
                                            None, None, w.scale)
        assert rflags == 0
        for name, a, b in [("dq", gq[:, sl], rq), ("dk", gk[:, sl], rk), ("dv", gv[:, sl], rv)]:
            assert_parity(a, b, w.dtype, f"bwd-workload heads {h0}-{h0 + 3} {name}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_bwd_empty_key_or_query_ranges(dtype):
    """Lk = 0: every row is fully masked, dq = 0 and the flag is raised.
    Lq = 0: no query reaches any key, dk = dv = 0."""
    import masked_head_attention_amd as M
    import torch

    td = torch.float16 if dtype == "f16" else torch.float32
    q = torch.randn(2, 3, 40, 64, device="cuda").to(td)
    z = torch.zeros(2, 3, 0, 64, dtype=td, device="cuda")
    dq, dk, dv = M.bwd(q, z, z, torch.randn_like(q))
    assert M.get_flags(clear=True) == M.FLAG_FULLY_MASKED_ROW
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0
    k = torch.randn(2, 3, 50, 64, device="cuda").to(td)
    e = torch.zeros(2, 3, 0, 64, dtype=td, device="cuda")
    dq, dk, dv = M.bwd(e, k, k.clone(), e, kind=M.CAUSAL)
    assert M.get_flags(clear=True) == 0
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_noncausal_long_rows_sampled():
    """No mask, bfloat16, L = 1024, D = 128: two heads against the oracle."""
    w = W.make("bwd-long", "bf16", 1, 4, 1024, 1024, 128, seed=61)
    g = W.grad_output(w)
    gq, gk, gv, flags = _run(w, g)
    assert flags == 0
    for h in (0, 3):
        sl = slice(h, h + 1)
        rq, rk, rv, _ = oracle.mha_bwd(w.f64("q")[:, sl], w.f64("k")[:, sl], w.f64("v")[:, sl],
                                       W.to_f64(g, w.dtype)[:, sl], 0, None, None, w.scale)
        for name, a, b in [("dq", gq[:, sl], rq), ("dk", gk[:, sl], rk), ("dv", gv[:, sl], rv)]:
            assert_parity(a, b, w.dtype, f"bwd-long head {h} {name}")


@pytest.mark.parametrize("B,H,L", [(3, 15, 1024), (1, 40, 2048)])
def test_bwd_block_map_covers_every_block(B, H, L):
    """Both kernels map workgroups to (head, block group) so that every block
    of a head stays on one XCD and an XCD's workgroups go in block-group order
    (longest causal groups first), with the heads past the last group of 8 in
    plain order. Each block's gradients do not depend on which workgroup
    computes them, so the whole call must equal one call per head bit for
    bit: a block computed twice or never would not. One head of the mapped
    part is also checked against the oracle."""
    import masked_head_attention_amd as M
    import torch

    w = W.make("bwd-map", "f16", B, H, L, L, 64, kind=W.CAUSAL | W.PADDING, seed=71,
               lens_range=(300, L))
    g = W.grad_output(w)
    gq, gk, gv, flags = _run(w, g)
    assert flags == 0
    q, k, v, go = (to_dev(a, w.dtype) for a in (w.q, w.k, w.v, g))
    lens = to_dev(w.lens, w.dtype)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            one = M.bwd(*(t[sl].contiguous() for t in (q, k, v)), go[sl].contiguous(),
                        mask=lens[b:b + 1].contiguous(), kind=w.kind, scale=w.scale)
            for name, whole, part in zip(("dq", "dk", "dv"), (gq, gk, gv), one):
                assert np.array_equal(whole[sl], from_dev(part)), (b, h, name)
    assert M.get_flags(clear=True) == 0
    bh = 33  # in the mapped part (complete groups of 8 heads) of both shapes
    b, h = divmod(bh, H)
    sl = (slice(b, b + 1), slice(h, h + 1))
    rq, rk, rv, _ = oracle.mha_bwd(w.f64("q")[sl], w.f64("k")[sl], w.f64("v")[sl],
                                   W.to_f64(g, w.dtype)[sl], w.kind, w.lens[b:b + 1], None,
                                   w.scale)
    for name, a, r in [("dq", gq[sl], rq), ("dk", gk[sl], rk), ("dv", gv[sl], rv)]:
        assert_parity(a, r, w.dtype, f"bwd-map head {bh} {name}")
    del torch


def test_bwd_f32_long_ragged_rows():
    """float32 at L = 517 (eight full 64-key chunks and a ragged one), D = 128,
    causal with padding lengths, against the oracle everywhere."""
    w = W.make("bwd-f32-long", "f32", 1, 2, 517, 517, 128, kind=W.CAUSAL | W.PADDING, seed=81,
               lens_range=(200, 517))
    _check(w, "bwd-f32-long")


BWD_KINDS = [0, W.CAUSAL, W.PADDING, W.CAUSAL | W.PADDING, W.ADDITIVE, W.ADDITIVE | W.CAUSAL,
             W.KEEP, W.ADDITIVE | W.PER_HEAD]


def _bwd_random_shapes(n=16, seed=4048):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        dtype = ["f32", "f16", "bf16"][c % 3]
        D = [16, 32, 64, 128][int(rng.integers(4))]
        kind = BWD_KINDS[int(rng.integers(len(BWD_KINDS)))]
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 11))
        Lq, Lk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        cases.append((dtype, D, kind, B, H, Lq, Lk, 500 + c))
    return cases


@pytest.mark.parametrize("dtype,D,kind,B,H,Lq,Lk,seed", _bwd_random_shapes())
def test_bwd_random_shapes(dtype, D, kind, B, H, Lq, Lk, seed):
    """Seeded random shapes for both kernels: odd tile counts (a wave pair's
    last step with one tile), Lq != Lk (also under the causal mask), head
    counts below and above a group of 8 (both branches of the workgroup map),
    every element type and head size, and the mask kinds."""
    w = W.make("bwd-rand", dtype, B, H, Lq, Lk, D, kind=kind, seed=seed,
               lens_range=(0, Lk) if kind & (W.PADDING | W.ADDITIVE | W.KEEP) else None,
               block_p=0.2 if kind & (W.ADDITIVE | W.KEEP) else 0.0, block=16)
    _check(w, f"bwd-rand-{dtype}-D{D}-k{kind}-{B}x{H}x{Lq}x{Lk}")
