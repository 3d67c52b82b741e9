"""GPU parity of mha_prenorm_cross_fwd_ws, the pre-LN cross-attention call
with a workspace. For bfloat16 calls without a mask tensor it copies K and V
to float16 once per call and runs the attention kernel on the copies, except
for heads holding a value float16 cannot represent (|x| > 65504), which run
on the bfloat16 tensors as the call without a workspace does.

Bar: the oracle's (unrounded pre-LN) output within 2e-3 + half an output ulp
elementwise; flags equal; heads that take the bfloat16 path equal the call
without a workspace bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from helpers import (TOL, assert_parity, from_dev, gpu_inputs, half_ulp, prenorm_workspace,
                     run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

CAUSAL, PADDING, ADDITIVE = W.CAUSAL, W.PADDING, W.ADDITIVE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_head_attention_amd as M

    M.init()
    M.get_flags(clear=True)
    yield


def _case(D, kind, H=4, B=2, Lq=150, Lk=300, seed=0, dtype="bf16"):
    return W.make("prenorm-ws", dtype, B=B, H=H, Lq=Lq, Lk=Lk, D=D, kind=kind, seed=seed,
                  lens_range=(40, Lk) if kind & (PADDING | ADDITIVE) else None,
                  block_p=0.1 if kind & ADDITIVE else 0.0, prenorm=True, x_mean=0.5,
                  x_std=3.0, residual=True)


def _ws_vs_oracle(w, what):
    print(f"[prenorm-ws] {what}: B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} D{w.D} kind{w.kind} "
          f"seed{w.seed}", flush=True)
    out, flags = run_gpu(w, workspace=prenorm_workspace(w))
    ref, rflags = run_oracle(w)
    assert_parity(from_dev(out), ref, w.dtype, what)
    assert flags == rflags, (what, flags, rflags)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", [0, CAUSAL, PADDING, CAUSAL | PADDING])
def test_ws_parity(D, kind):
    """Four heads per workgroup, ragged query and key counts (several tiles
    and a partial one), every mask kind the copies serve."""
    _ws_vs_oracle(_case(D, kind, seed=300 + D + kind), f"ws-D{D}-k{kind}")


@pytest.mark.parametrize("H,Lq,Lk", [(1, 97, 65), (2, 200, 130), (3, 33, 257), (6, 129, 64)])
def test_ws_head_groups(H, Lq, Lk):
    """Head groups of one and two heads (H not a multiple of 4), a single key
    tile, a key count one past a tile, a query count one past a block."""
    _ws_vs_oracle(_case(64, 0, H=H, Lq=Lq, Lk=Lk, seed=400 + H), f"ws-H{H}-Lq{Lq}-Lk{Lk}")


@pytest.mark.parametrize("D,kind", [(64, 0), (128, CAUSAL), (32, PADDING)])
def test_ws_heads_beyond_float16(D, kind):
    """Values above float16's range in some heads only: those heads (and only
    those) take the bfloat16 kernel, whose result is the call without a
    workspace bit for bit; every head matches the oracle."""
    w = _case(D, kind, seed=500 + D)
    k = W.bf16_bits_to_f32(w.k).astype(np.float64)
    v = W.bf16_bits_to_f32(w.v).astype(np.float64)
    k[0, 1, 10, 3] = 7.0e4          # head (0, 1): a key
    v[1, 2, 200, D - 1] = -3.0e5    # head (1, 2): a value
    v[1, 3, 5, 0] = 6.6e4           # head (1, 3): just above float16's largest finite value
    w.k = W.round_to(k, "bf16")
    w.v = W.round_to(v, "bf16")
    d = gpu_inputs(w)
    out_ws, flags_ws = run_gpu(w, inputs=d, workspace=prenorm_workspace(w))
    out_plain, flags_plain = run_gpu(w, inputs=d)
    ref, rflags = run_oracle(w)
    got = from_dev(out_ws)
    plain = from_dev(out_plain)
    assert flags_ws == rflags and flags_plain == rflags
    assert np.isfinite(got).all()
    # the bar of the bfloat16 path with large values: tol + half an output ulp
    # + 2^-14 max|V| of the head (P carried with about 16 significant bits)
    vmax = np.abs(w.f64("v")).max(axis=(2, 3))  # [B, H]
    scale_bh = np.repeat(vmax[:, None, :], w.Lq, axis=1).repeat(w.D, axis=2)
    allowed = TOL["bf16"] + half_ulp(ref, "bf16") + 2.0 ** -14 * scale_bh
    err = np.abs(got - ref)
    assert (err <= allowed).all(), float((err / allowed).max())
    for b, h in [(0, 1), (1, 2), (1, 3)]:
        cols = slice(h * D, (h + 1) * D)
        assert np.array_equal(got[b, :, cols], plain[b, :, cols]), (b, h)


@pytest.mark.parametrize("D,kind,Lk", [(64, PADDING, 384), (128, 0, 257), (32, PADDING, 500),
                                       (64, CAUSAL | PADDING, 512)])
def test_ws_remapped_grids(D, kind, Lk):
    """Grids of 32 workgroups (B=4, two groups of 4 heads, 4 query blocks):
    without a causal mask a grid that is a multiple of 8 takes the remap that
    keeps a head group's query blocks on one XCD, so each workgroup's batch
    entry, head group and length come from the remapped index."""
    w = _case(D, kind, H=8, B=4, Lq=512, Lk=Lk, seed=1000 + D + kind)
    _ws_vs_oracle(w, f"ws-grid32-D{D}-k{kind}-Lk{Lk}")


def test_ws_sizes_errors_and_ignored_workspaces():
    """The size query, a short or misaligned workspace (MHA_E_WORKSPACE), and
    calls that ignore the workspace (float16, a mask tensor): those equal the
    call without one bit for bit."""
    import torch

    import masked_head_attention_amd as M

    B, H, Lq, Lk, D = 2, 4, 150, 300, 64
    need = M.prenorm_cross_workspace_size(B, H, Lq, Lk, D, M.BF16)
    kv = (B * H * Lk * D * 2 + 255) // 256 * 256
    assert need == 2 * kv + (B * H * 16 + 255) // 256 * 256 + (B * Lq * 8 + 255) // 256 * 256
    assert M.prenorm_cross_workspace_size(B, H, Lq, Lk, D, M.F16) == 0
    assert M.prenorm_cross_workspace_size(B, H, Lq, Lk, D, M.F32) == 0
    assert M.prenorm_cross_workspace_size(B, H, Lq, 0, D, M.BF16) == 0

    w = _case(D, 0, B=B, H=H, Lq=Lq, Lk=Lk, seed=600)
    d = gpu_inputs(w)
    short = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MhaError) as e:
        run_gpu(w, inputs=d, workspace=short)
    assert e.value.status == 11
    big = torch.zeros(need + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MhaError) as e:
        run_gpu(w, inputs=d, workspace=big[8:8 + need])
    assert e.value.status == 11
    torch.cuda.synchronize()

    tiny = torch.zeros(1, dtype=torch.uint8, device="cuda")
    for ww in (_case(D, 0, B=B, H=H, Lk=Lk, seed=601, dtype="f16"),
               _case(D, ADDITIVE, B=B, H=H, Lk=Lk, seed=602)):
        dd = gpu_inputs(ww)
        a, fa = run_gpu(ww, inputs=dd, workspace=tiny)
        b, fb = run_gpu(ww, inputs=dd)
        assert fa == fb
        assert torch.equal(a, b)


def test_ws_reuse_is_deterministic():
    """One workspace shared by calls on different inputs, one after another:
    each call gives what it gives with a fresh workspace."""
    import torch

    w1 = _case(64, CAUSAL, seed=700)
    w2 = _case(64, PADDING, seed=701)
    ws = prenorm_workspace(w1)
    d1, d2 = gpu_inputs(w1), gpu_inputs(w2)
    a1, _ = run_gpu(w1, inputs=d1, workspace=ws)
    a2, _ = run_gpu(w2, inputs=d2, workspace=ws)
    b1, _ = run_gpu(w1, inputs=d1, workspace=ws)
    c2, _ = run_gpu(w2, inputs=d2, workspace=prenorm_workspace(w2))
    assert torch.equal(a1, b1)
    assert torch.equal(a2, c2)


@pytest.mark.parametrize("garbage", ["nan", "nan-inf"])
@pytest.mark.parametrize("D", [64, 128])
def test_ws_nonfinite_padding_rows_do_not_leak(garbage, D):
    """Key rows at or past a sequence's length do not take part [MMHA 3.1].
    NaN there is copied to float16 and never read (the attention kernel's
    buffers end at the length); an infinity flags its head, which then takes
    the bfloat16 kernel, which never reads it either. No NONFINITE flag."""
    w = _case(D, PADDING, B=3, H=4, Lq=90, Lk=200, seed=800 + D)
    w.lens = np.array([37, 130, 1], np.int32)
    for name in ("k", "v"):
        a = w.f64(name).copy()
        for b, L in enumerate(w.lens):
            a[b, :, L::2] = np.nan
            a[b, :, L + 1::2] = np.inf if garbage == "nan-inf" else np.nan
        setattr(w, name, W.round_to(a, "bf16"))
    _ws_vs_oracle(w, f"ws-pad-garbage-{garbage}-D{D}")


def _ws_random_cases(n=10, seed=4242):
    rng = np.random.default_rng(seed)
    kinds = [0, CAUSAL, PADDING, CAUSAL | PADDING]
    out = []
    for i in range(n):
        out.append((int(rng.choice([16, 32, 64, 128])), int(rng.choice(kinds)),
                    int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 300)),
                    int(rng.integers(1, 300)), 900 + i))
    return out


@pytest.mark.parametrize("D,kind,B,H,Lq,Lk,seed", _ws_random_cases())
def test_ws_random_shapes(D, kind, B, H, Lq, Lk, seed):
    """Seeded random shapes: head groups of 1, 2 and 4, ragged query and key
    counts (one key to several tiles), every mask kind the copies serve."""
    w = W.make("prenorm-ws-rand", "bf16", B=B, H=H, Lq=Lq, Lk=Lk, D=D, kind=kind, seed=seed,
               lens_range=(0, Lk) if kind & PADDING else None, prenorm=True, x_mean=0.5,
               x_std=3.0, residual=True)
    _ws_vs_oracle(w, f"ws-rand-{seed}")
