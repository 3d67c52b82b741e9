"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bar: |gpu - oracle| <= tol + half an output ulp elementwise, tol = 1e-5 for
float32 and 2e-3 for float16/bfloat16; flags, tile skip counts and mask
decisions must agree exactly.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import (TOL, assert_parity, from_dev, gpu_inputs, half_ulp, prenorm_workspace,
                     run_gpu, run_oracle, to_dev)

pytestmark = pytest.mark.gpu

CAUSAL, PADDING, ADDITIVE = W.CAUSAL, W.PADDING, W.ADDITIVE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_head_attention_amd as M

    M.init()
    yield
    M.set_debug_counters(None)


def _check(w, what):
    print(f"[parity] {what}: {w.name} {w.dtype} B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} D{w.D} "
          f"kind{w.kind} seed{w.seed}", flush=True)
    out_t, flags = run_gpu(w)
    ref, rflags = run_oracle(w)
    err = assert_parity(from_dev(out_t), ref, w.dtype, what)
    assert flags == rflags, (what, flags, rflags)
    return err


# ---- the five workloads at reduced sizes (full elementwise check) ----------
REDUCED = {
    1: dict(),
    2: dict(),  # full size is small enough for a full oracle pass
    3: dict(H=2, Lq=300, Lk=300),
    4: dict(B=2, H=4, Lq=200, Lk=150),
    5: dict(B=3, H=2, Lq=200, Lk=200, lens_range=(30, 200), block_p=0.3),
}


@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_workload_reduced(cfg):
    _check(W.config(cfg, **REDUCED[cfg]), f"cfg{cfg}-reduced")


# ---- the sweep: every dtype x D x mask kind, ragged sizes -------------------
KINDS = [0, CAUSAL, PADDING, CAUSAL | PADDING, ADDITIVE, CAUSAL | ADDITIVE]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", KINDS)
def test_sweep(dtype, D, kind):
    w = W.make("sweep", dtype, B=2, H=2, Lq=75, Lk=141, D=D, kind=kind, seed=D + 7 * kind,
               lens_range=(1, 141) if kind & (PADDING | ADDITIVE) else None,
               block_p=0.25 if kind & ADDITIVE else 0.0, block=16)
    _check(w, f"sweep-{dtype}-D{D}-k{kind}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kind", [0, CAUSAL, PADDING, ADDITIVE])
def test_prenorm_sweep(dtype, kind):
    w = W.make("prenorm-sweep", dtype, B=2, H=3, Lq=70, Lk=99, D=64, kind=kind, seed=11 + kind,
               lens_range=(5, 99) if kind & (PADDING | ADDITIVE) else None,
               block_p=0.2 if kind & ADDITIVE else 0.0, block=16, prenorm=True, x_mean=0.5,
               x_std=3.0, residual=(kind != PADDING))
    _check(w, f"prenorm-{dtype}-k{kind}")


def _random_shapes(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        dtype = ["f32", "f16", "bf16"][c % 3]
        D = [16, 32, 64, 128][int(rng.integers(4))]
        kind = KINDS[int(rng.integers(len(KINDS)))]
        prenorm = bool(c % 4 == 3) and not (kind & ADDITIVE and kind & CAUSAL)
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        Lq, Lk = int(rng.integers(1, 260)), int(rng.integers(1, 260))
        if c % 5 == 0:
            Lq, Lk = max(Lq, Lk), min(Lq, Lk)  # more queries than keys
        cases.append((dtype, D, kind, prenorm, B, H, Lq, Lk, 100 + c))
    return cases


@pytest.mark.parametrize("dtype,D,kind,prenorm,B,H,Lq,Lk,seed", _random_shapes())
def test_random_shapes(dtype, D, kind, prenorm, B, H, Lq, Lk, seed):
    """Seeded random shapes: Lq > Lk with causal, single heads, two- and
    three-head pre-LN groups, lengths of 1."""
    w = W.make("rand", dtype, B=B, H=H, Lq=Lq, Lk=Lk, D=D, kind=kind, seed=seed,
               lens_range=(0, Lk) if kind & (PADDING | ADDITIVE) else None,
               block_p=0.2 if kind & ADDITIVE else 0.0, block=16, prenorm=prenorm,
               x_mean=0.5, x_std=2.0, residual=prenorm)
    _check(w, f"rand-{dtype}-D{D}-k{kind}-pre{int(prenorm)}-{B}x{H}x{Lq}x{Lk}")


# ---- the extra mask forms: keep-masks and per-head mask tensors --------------
KEEP, PER_HEAD = W.KEEP, W.PER_HEAD
MASK_FORMS = [KEEP, KEEP | CAUSAL, ADDITIVE | PER_HEAD, KEEP | PER_HEAD,
              ADDITIVE | PER_HEAD | CAUSAL]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("kind", MASK_FORMS)
def test_mask_forms(dtype, D, kind):
    w = W.make("mask-form", dtype, B=2, H=3, Lq=75, Lk=141, D=D, kind=kind, seed=D + kind,
               lens_range=(1, 141), block_p=0.25, block=16)
    _check(w, f"mask-form-{dtype}-D{D}-k{kind}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kind", [KEEP | PER_HEAD, ADDITIVE | PER_HEAD, KEEP | CAUSAL])
def test_prenorm_mask_forms(dtype, kind):
    # H = 8: the 16-bit kernel serves groups of 4 heads, each with its own slab
    w = W.make("prenorm-mask-form", dtype, B=2, H=8, Lq=70, Lk=99, D=32, kind=kind, seed=kind,
               lens_range=(5, 99), block_p=0.2, block=16, prenorm=True, x_mean=0.5,
               x_std=3.0, residual=True)
    _check(w, f"prenorm-mask-form-{dtype}-k{kind}")


def test_keep_unaligned_rows_and_counters():
    import torch
    import masked_head_attention_amd as M

    w = W.make("keep-odd-lk", "f16", B=2, H=2, Lq=67, Lk=203, D=64, kind=KEEP | PER_HEAD | CAUSAL,
               seed=9, lens_range=(50, 203), block_p=0.3, block=32)
    _check(w, "keep-odd-Lk")
    rows, keys = M.tile_config(1, w.D, w.kind)
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda")
    M.set_debug_counters(cnt)
    try:
        run_gpu(w)
        torch.cuda.synchronize()
    finally:
        M.set_debug_counters(None)
    comp, skip = oracle.tile_counts(w.kind, w.B, w.H, w.Lq, w.Lk, rows, keys, w.lens,
                                    w.f64("add"))
    full = oracle.fully_masked_rows(w.kind, w.B, w.H, w.Lq, w.Lk, w.lens, w.f64("add"))
    assert cnt.tolist() == [comp, skip, full], (cnt.tolist(), comp, skip, full)


def test_unaligned_additive_rows():
    """Lk * 2 bytes not a multiple of 16: the additive mask rows are read
    element by element."""
    w = W.make("odd-lk", "f16", B=2, H=2, Lq=67, Lk=203, D=64, kind=ADDITIVE | CAUSAL, seed=3,
               lens_range=(50, 203), block_p=0.3, block=32)
    _check(w, "additive-odd-Lk")


# ---- full sizes, in the benchmark's launch configuration -------------------
def _nan_out(w):
    """An output buffer pre-filled with NaN, so a row the kernel never writes
    fails the comparison."""
    import torch

    from helpers import torch_dtype

    shape = (w.B, w.Lq, w.H * w.D) if w.prenorm else (w.B, w.H, w.Lq, w.D)
    return torch.full(shape, float("nan"), dtype=torch_dtype(w.dtype), device="cuda")


@pytest.mark.parametrize("cfg,ws", [(1, False), (2, False), (3, False), (4, False), (4, True),
                                    (5, False)])
def test_workload_full_size_elementwise(cfg, ws):
    """Every output element of the full-size workload against the fp64 oracle
    (the whole grid, including the XCD workgroup remap and the heaviest-first
    causal order). The pre-LN cross-attention workload (B=32, H=16,
    Lq=Lk=2048, D=64, bfloat16) is compared against the unrounded oracle,
    with and without a workspace (the benchmark times the workspace call)."""
    w = W.config(cfg)
    print(f"[parity] full-size cfg{cfg} {w.name} elementwise, workspace {ws}", flush=True)
    wsp = prenorm_workspace(w) if ws else None
    out_t, flags = run_gpu(w, out=_nan_out(w), workspace=wsp)
    del wsp
    got = from_dev(out_t)
    del out_t
    ref, rflags = run_oracle(w)
    assert_parity(got, ref, w.dtype, f"cfg{cfg}-full")
    assert flags == rflags


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind,prenorm", [(PADDING, False), (CAUSAL | PADDING, False),
                                          (PADDING, True)])
def test_nonfinite_padding_rows_do_not_leak(dtype, D, kind, prenorm):
    """Key rows at or past a sequence's length do not take part [MMHA 3.1],
    whatever the memory there holds: K/V rows >= len_b filled with NaN, +inf
    and -inf must leave every output equal to the oracle's (which never reads
    them), with no NONFINITE flag. Lengths fall inside tiles, so edge tiles
    straddle the garbage."""
    w = W.make("pad-garbage", dtype, B=3, H=2, Lq=90, Lk=200, D=D, kind=kind, seed=31 + D,
               lens_range=(1, 200), prenorm=prenorm, x_mean=0.5, x_std=3.0, residual=prenorm)
    w.lens = np.array([37, 130, 1], np.int32)
    for name in ("k", "v"):
        a = w.f64(name).copy()
        for b, L in enumerate(w.lens):
            a[b, :, L::3] = np.nan
            a[b, :, L + 1::3] = np.inf
            a[b, :, L + 2::3] = -np.inf
        setattr(w, name, W.round_to(a, dtype))
    assert not np.isfinite(w.f64("v")).all()
    _check(w, f"pad-garbage-{dtype}-D{D}-k{kind}-pre{int(prenorm)}")


# ---- exact decisions: skip counters and the mask probe ---------------------
@pytest.mark.parametrize("cfg,over", [(2, {}), (3, dict(H=2, Lq=700, Lk=700)),
                                      (5, dict(B=4, H=2)), (1, {}),
                                      # 16-bit causal runs two key splits per query
                                      # block; zero lengths make fully masked rows
                                      (3, dict(B=3, H=2, Lq=300, Lk=300, D=64,
                                               kind=CAUSAL | PADDING, lens_range=(0, 2))),
                                      (3, dict(B=2, H=2, Lq=260, Lk=260, D=128, dtype="bf16",
                                               kind=CAUSAL | PADDING, lens_range=(0, 1)))])
def test_skip_counters_match_oracle(cfg, over):
    import torch
    import masked_head_attention_amd as M

    w = W.config(cfg, **over)
    rows, keys = M.tile_config({"f32": 0, "f16": 1, "bf16": 2}[w.dtype], w.D, w.kind)
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda")
    M.set_debug_counters(cnt)
    try:
        run_gpu(w)
        torch.cuda.synchronize()
    finally:
        M.set_debug_counters(None)
    comp, skip = oracle.tile_counts(w.kind, w.B, w.H, w.Lq, w.Lk, rows, keys, w.lens,
                                    w.f64("add"))
    full = oracle.fully_masked_rows(w.kind, w.B, w.H, w.Lq, w.Lk, w.lens, w.f64("add"))
    assert cnt.tolist() == [comp, skip, full], (cnt.tolist(), comp, skip, full)


@pytest.mark.parametrize("dtype,kind,D", [("f16", ADDITIVE, 64), ("f16", CAUSAL, 128),
                                          ("f32", CAUSAL | PADDING, 64),
                                          ("bf16", ADDITIVE | CAUSAL, 32)])
def test_mask_probe_bitmap(dtype, kind, D):
    """Q = 0 and V one-hot over key block r: out[i, d] = legal(i, rD + d) / n_i,
    so Lk/D runs read back the whole mask bitmap, compared bit for bit."""
    import torch

    L = 256
    w = W.make("probe", dtype, B=2, H=1, Lq=L, Lk=L, D=D, kind=kind, seed=5,
               lens_range=(40, L), block_p=0.3 if kind & ADDITIVE else 0.0, block=32)
    dec = oracle.mask_decisions(kind, w.B, L, L, w.lens, w.f64("add")).astype(bool)
    n = (~dec).sum(axis=2)
    d = gpu_inputs(w)
    d["q"] = torch.zeros_like(d["q"])
    d["k"] = torch.zeros_like(d["k"])
    got = np.zeros((w.B, L, L), bool)
    for r in range(L // D):
        v = np.zeros((w.B, 1, L, D), np.float32)
        for j in range(D):
            v[:, 0, r * D + j, j] = 1.0
        d["v"] = to_dev(W.round_to(v, dtype), dtype)
        out, _ = run_gpu(w, inputs=d)
        o = from_dev(out)[:, 0]  # [B, L, D] = legal / n
        got[:, :, r * D:(r + 1) * D] = o * np.maximum(n, 1)[:, :, None] > 0.5
    assert np.array_equal(got, ~dec)


# ---- closed forms and special cases on the GPU ------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_causal_row0_is_v0_exactly(dtype):
    w = W.make("row0", dtype, B=2, H=3, Lq=100, Lk=100, D=64, kind=CAUSAL, seed=1)
    out, _ = run_gpu(w)
    o = from_dev(out)
    assert np.array_equal(o[:, :, 0, :], w.f64("v")[:, :, 0, :])


def test_q_zero_gives_prefix_means():
    import torch

    w = W.make("qzero", "f16", B=1, H=2, Lq=300, Lk=300, D=128, kind=CAUSAL | PADDING, seed=4,
               lens_range=(100, 250))
    d = gpu_inputs(w)
    d["q"] = torch.zeros_like(d["q"])
    out, _ = run_gpu(w, inputs=d)
    v = w.f64("v")
    ref = np.zeros_like(v[:, :, :w.Lq])
    for b in range(w.B):
        for i in range(w.Lq):
            nkeys = min(i, w.lens[b] - 1) + 1
            ref[b, :, i] = v[b, :, :nkeys].mean(axis=1)
    assert_parity(from_dev(out), ref, "f16", "q=0 prefix means")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("z", [88.0, -88.0, 11.0])
def test_two_key_logistic_large_logits(dtype, z):
    """Logits +-z on two keys (scale 1): o = sigma(2z) v0 + (1 - sigma(2z)) v1,
    finite even where exp(z) alone would overflow fp16/fp32."""
    import torch
    import masked_head_attention_amd as M

    D = 16
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    q = torch.zeros(1, 1, 1, D, dtype=td, device="cuda")
    q[..., 0] = z
    k = torch.zeros(1, 1, 2, D, dtype=td, device="cuda")
    k[0, 0, 0, 0], k[0, 0, 1, 0] = 1.0, -1.0
    v = torch.zeros(1, 1, 2, D, dtype=td, device="cuda")
    v[0, 0, 0, :], v[0, 0, 1, :] = 3.0, -2.0
    M.get_flags(clear=True)
    out = M.fwd(q, k, v, scale=1.0)
    assert M.get_flags() == 0
    sig = 1.0 / (1.0 + math.exp(-2 * z))
    ref = np.full((1, 1, 1, D), sig * 3.0 - 2.0 * (1 - sig))
    assert_parity(from_dev(out), ref, dtype, f"two-key z={z}")


def test_fully_masked_rows_zero_and_flag():
    import torch
    import masked_head_attention_amd as M

    w = W.make("fm", "f16", B=3, H=2, Lq=50, Lk=64, D=64, kind=PADDING, seed=2,
               lens_range=(0, 0))
    w.lens = np.array([0, 64, 10], np.int32)
    out, flags = run_gpu(w)
    o = from_dev(out)
    assert np.all(o[0] == 0.0)
    assert flags == M.FLAG_FULLY_MASKED_ROW
    ref, rflags = run_oracle(w)
    assert_parity(o, ref, "f16", "fully masked")
    # lengths outside [0, Lk] act clamped and raise BAD_LENGTH
    w.lens = np.array([-5, 100, 10], np.int32)
    out, flags = run_gpu(w)
    ref, rflags = run_oracle(w)
    assert flags == rflags == (M.FLAG_FULLY_MASKED_ROW | M.FLAG_BAD_LENGTH)
    assert_parity(from_dev(out), ref, "f16", "bad lengths")


def test_prenorm_fully_masked_row_stores_residual():
    w = W.make("pre-fm", "bf16", B=2, H=2, Lq=40, Lk=40, D=32, kind=PADDING, seed=8,
               lens_range=(0, 0), prenorm=True, x_mean=0.5, x_std=3.0, residual=True)
    w.lens = np.array([0, 17], np.int32)
    out, flags = run_gpu(w)
    o = from_dev(out)
    assert np.array_equal(o[0], w.f64("x")[0])
    assert flags == 1


def test_nonfinite_flag():
    import torch

    w = W.make("nan", "f32", B=1, H=2, Lq=40, Lk=40, D=32, kind=0, seed=9)
    d = gpu_inputs(w)
    d["v"][0, 1, 7, 3] = float("nan")
    out, flags = run_gpu(w, inputs=d)
    assert flags == 2
    o = from_dev(out)
    assert np.isnan(o[0, 1, :, 3]).all() and np.isfinite(o[0, 0]).all()


def test_empty_and_degenerate_shapes():
    import torch
    import masked_head_attention_amd as M

    # Lk = 0: every row fully masked
    q = torch.randn(1, 2, 5, 64, device="cuda", dtype=torch.float16)
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.float16)
    M.get_flags(clear=True)
    out = M.fwd(q, k, k.clone(), kind=CAUSAL)
    assert torch.count_nonzero(out).item() == 0 and M.get_flags() == M.FLAG_FULLY_MASKED_ROW
    # Lq = 0 and B = 0: nothing to do
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.float16)
    kk = torch.randn(1, 2, 9, 64, device="cuda", dtype=torch.float16)
    assert M.fwd(q0, kk, kk).shape == (1, 2, 0, 64)
    qb = torch.empty(0, 2, 4, 64, device="cuda", dtype=torch.float16)
    assert M.fwd(qb, torch.empty(0, 2, 4, 64, device="cuda", dtype=torch.float16),
                 torch.empty(0, 2, 4, 64, device="cuda", dtype=torch.float16)).numel() == 0
    # single query, single key
    w = W.make("1x1", "bf16", B=1, H=1, Lq=1, Lk=1, D=128, kind=CAUSAL, seed=1)
    _check(w, "1x1")
    # Lq != Lk with causal (top-left aligned)
    w = W.make("rect", "f16", B=2, H=2, Lq=130, Lk=37, D=32, kind=CAUSAL, seed=6)
    _check(w, "rect-causal")


def test_repeat_calls_are_deterministic():
    w = W.config(5, B=2, H=2)
    d = gpu_inputs(w)
    a, _ = run_gpu(w, inputs=d)
    b, _ = run_gpu(w, inputs=d)
    assert np.array_equal(from_dev(a), from_dev(b))


def test_graph_replays_match_eager():
    """Launches captured in a HIP graph give the eager result on every replay,
    with eager work and synchronisations between the replays."""
    import torch
    import masked_head_attention_amd as M

    w = W.config(5, B=2, H=2)
    d = gpu_inputs(w)
    eager, _ = run_gpu(w, inputs=d)
    eager = eager.clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            M.fwd(d["q"], d["k"], d["v"], mask=d["mask"], kind=w.kind, scale=w.scale, out=out)
    for r in range(4):
        out.fill_(float("nan"))
        _ = torch.randn(1000, device="cuda").sum()  # unrelated eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"


@pytest.mark.parametrize("kind,D", [(0, 64), (CAUSAL, 128), (ADDITIVE, 64)])
def test_bf16_prenorm_keys_beyond_f16_range(kind, D):
    """Pre-LN, bfloat16: landed K tiles are rewritten into float16 for a
    float16 Q K^T product, except tile 0 of a head, which multiplies the
    float16 query in two exact bfloat16 parts. A tile holding a finite
    |k| > 65504 must be fetched again and take that split product. Large
    keys sit in tile 0, in tile 2 and (just above float16's range) in tile 3.
    The query's float16 rounding moves a score by about 2^-12 |q_d k_d|, so
    it stays small wherever the outlier's score is not far beyond the rest."""
    w = W.make("bf16-big-k", "bf16", B=2, H=2, Lq=150, Lk=300, D=D, kind=kind, seed=9 + D + kind,
               lens_range=(40, 300) if kind & ADDITIVE else None, block_p=0.1, block=16,
               prenorm=True, x_mean=0.5, x_std=3.0, residual=True)
    k = W.bf16_bits_to_f32(w.k).astype(np.float64)
    k[0, 0, 10, 3] = 7.0e4           # tile 0 of (b0, h0)
    k[0, 1, 140, 0] = -9.0e4         # tile 2 of (b0, h1)
    k[1, 1, 200, D - 1] = 6.6e4      # tile 3 of (b1, h1), just above float16's largest value
    w.k = W.round_to(k, "bf16")
    _check(w, f"bf16-big-k-k{kind}-D{D}")


@pytest.mark.parametrize("kind,D,prenorm", [(0, 64, False), (CAUSAL, 64, False), (0, 64, True),
                                            (CAUSAL | PADDING, 32, False)])
def test_bf16_values_beyond_f16_range(kind, D, prenorm):
    """bfloat16 V is rewritten into float16 for the P V product where it fits;
    a tile holding a finite value above float16's range (65504) must take the
    split-P bfloat16 path and still match the oracle. Large values sit in
    some tiles only, so both paths run in one call."""
    w = W.make("bf16-big-v", "bf16", B=2, H=2, Lq=150, Lk=300, D=D, kind=kind, seed=5 + D,
               lens_range=(40, 300) if kind & PADDING else None, prenorm=prenorm, x_mean=0.5,
               x_std=3.0, residual=prenorm)
    v = W.bf16_bits_to_f32(w.v).astype(np.float64)
    v[0, 0, 70, 3] = 3.0e5          # tile 1 of (b0, h0)
    v[0, 0, 200, D - 1] = -1.0e6    # tile 3 of (b0, h0)
    v[1, 1, 5, 0] = 7.0e4           # just above float16's largest finite value
    w.v = W.round_to(v, "bf16")
    what = f"bf16-big-v-k{kind}-D{D}-pre{int(prenorm)}"
    print(f"[parity] {what}", flush=True)
    out_t, flags = run_gpu(w)
    ref, rflags = run_oracle(w)
    got = from_dev(out_t)
    assert flags == rflags
    assert np.isfinite(got).all()
    # The bar: tol + half an output ulp, plus 2^-14 * max|V| of the head. With
    # V up to 1e6 the outputs reach ~1e3, where 2e-3 is below the rounding
    # noise of any bf16 P V product: P is carried with ~16 significant bits
    # (hi + lo parts), so a term's error is <= 2^-16 |P_k V_k|; an output near
    # a bf16 rounding midpoint then lands on either side. A tile that took the
    # float16 path with such values would give inf or O(|V|) errors instead.
    vmax = np.abs(w.f64("v")).max(axis=(2, 3))  # [B, H]
    if prenorm:
        scale_bh = np.repeat(vmax[:, None, :], w.Lq, axis=1).repeat(w.D, axis=2)  # [B, Lq, H*D]
    else:
        scale_bh = vmax[:, :, None, None] * np.ones((1, 1, w.Lq, w.D))
    err = np.abs(got - ref)
    allowed = TOL["bf16"] + half_ulp(ref, "bf16") + 2.0 ** -14 * scale_bh
    assert (err <= allowed).all(), (what, float((err / allowed).max()))
