"""GPU parity of the decode call (one new query row per (batch, head) against
a key/value cache with per-sequence lengths, the inference-engine use of
"masked multi head attention" CUDA notes, section 6.1) against the fp64
oracle, through the C ABI.

Bar: outputs |gpu - oracle| <= tol + half an output ulp elementwise (tol 1e-5
for float32, 2e-3 for float16/bfloat16); the log-sum-exp, a float32 output
for every dtype, within LSE_TOL(lse) = 1e-5 + 1e-6 |lse| (float32 rounding of
the score sums and of the exponentials, relative 2^-24 per operation, over D
products and the key sum); flags agree exactly.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import assert_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


def lse_tol(ref):
    return 1e-5 + 1e-6 * np.abs(np.where(np.isfinite(ref), ref, 0.0))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_head_attention_amd as M

    M.init()
    M.get_flags(clear=True)
    yield


def _q3(w):
    return w.q.reshape(w.B, w.H, w.D)


def _run(w, lens=None, workspace=None):
    import masked_head_attention_amd as M

    lens = w.lens if lens is None else lens
    print(f"[decode] {w.name} {w.dtype} B{w.B} H{w.H} Lk{w.Lk} D{w.D} seed {w.seed}", flush=True)
    q = to_dev(_q3(w), w.dtype)
    k = to_dev(w.k, w.dtype)
    v = to_dev(w.v, w.dtype)
    ln = to_dev(lens, w.dtype) if lens is not None else None
    M.get_flags(clear=True)
    out, lse = M.decode(q, k, v, ln, scale=w.scale, workspace=workspace)
    flags = M.get_flags(clear=True)
    return from_dev(out), lse.cpu().numpy().astype(np.float64), flags


def _check(w, what, lens=None):
    got, glse, flags = _run(w, lens)
    lens = w.lens if lens is None else lens
    ref, rlse, rflags = oracle.decode(W.to_f64(_q3(w), w.dtype), w.f64("k"), w.f64("v"), lens,
                                      w.scale)
    assert_parity(got, ref, w.dtype, what)
    assert np.array_equal(np.isneginf(glse), np.isneginf(rlse)), what
    fin = np.isfinite(rlse)
    err = np.abs(glse[fin] - rlse[fin])
    assert np.all(err <= lse_tol(rlse[fin])), (what, float(err.max(initial=0.0)))
    assert flags == rflags, (what, flags, rflags)


def _work(dtype, B, H, Lk, D, seed, lens_range=None, std=1.0):
    kind = W.PADDING if lens_range is not None else 0
    return W.make(f"decode-{dtype}-{D}-{Lk}", dtype, B, H, 1, Lk, D, kind=kind, seed=seed,
                  lens_range=lens_range, qkv_std=std)


# one split per head (short caches) and split keys with the merge kernel
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("Lk", [1, 37, 700, 3001])
def test_decode_parity(dtype, D, Lk):
    w = _work(dtype, 3, 5, Lk, D, seed=Lk + D, lens_range=(0, Lk))
    _check(w, f"decode-{dtype}-D{D}-Lk{Lk}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_decode_no_lengths_many_splits(dtype):
    # two heads of a long cache: many splits per head, every key legal
    w = _work(dtype, 1, 2, 8192, 128, seed=21)
    _check(w, f"decode-nolens-{dtype}")


def test_decode_split_boundaries():
    """Lengths at, one below and one above the split chunk of the plan."""
    import masked_head_attention_amd as M

    B, H, Lk, D = 8, 2, 2048, 64
    need = M.decode_workspace_size(B, H, Lk, D, M.F16)
    assert need > 0
    nsplit = need // (B * H * (D + 2) * 4)
    chunk = -(-Lk // nsplit)
    lens = np.array([chunk - 1, chunk, chunk + 1, 2 * chunk, 1, 0, Lk - 1, Lk], np.int32)
    w = _work("f16", B, H, Lk, D, seed=22, lens_range=(0, Lk))
    _check(w, "decode-boundaries", lens=lens)


def test_decode_bad_lengths_flag_and_clamp():
    w = _work("f16", 4, 3, 300, 64, seed=23, lens_range=(0, 300))
    _check(w, "decode-bad-lengths", lens=np.array([-5, 301, 0, 7], np.int32))


def test_decode_large_logits():
    """float16 inputs whose scaled logits reach about +-88 (std 16): exp of
    them overflows float32 unless the running maximum is subtracted first."""
    w = _work("f16", 2, 4, 1500, 64, seed=24, lens_range=(1, 1500), std=4.0)
    got, glse, _ = _run(w)
    s = np.einsum("bhd,bhkd->bhk", W.to_f64(_q3(w), "f16"), w.f64("k")) * w.scale
    assert np.abs(s).max() > 60.0
    _check(w, "decode-large-logits")


def test_decode_empty_and_zero_length_cache():
    import masked_head_attention_amd as M
    import torch

    q = torch.zeros(0, 4, 64, dtype=torch.float16, device="cuda")
    k = torch.zeros(0, 4, 10, 64, dtype=torch.float16, device="cuda")
    M.decode(q, k, k)
    assert M.get_flags(clear=True) == 0
    q = torch.randn(2, 3, 64, device="cuda").half()
    k = torch.zeros(2, 3, 0, 64, dtype=torch.float16, device="cuda")
    out, lse = M.decode(q, k, k)
    assert M.get_flags(clear=True) == M.FLAG_FULLY_MASKED_ROW
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_decode_nonfinite_flag():
    import masked_head_attention_amd as M
    import torch

    q = torch.randn(2, 2, 64, device="cuda").half()
    k = torch.randn(2, 2, 5000, 64, device="cuda").half()
    v = torch.randn(2, 2, 5000, 64, device="cuda").half()
    v[1, 0, 4000, 3] = float("nan")
    out, _ = M.decode(q, k, v)
    assert M.get_flags(clear=True) == M.FLAG_NONFINITE
    o = out.float().cpu()
    assert torch.isnan(o[1, 0, 3]) and torch.isfinite(o[0]).all()


def test_decode_workspace_errors():
    import masked_head_attention_amd as M
    import torch

    q = torch.randn(4, 8, 128, device="cuda").half()
    k = torch.randn(4, 8, 4096, 128, device="cuda").half()
    need = M.decode_workspace_size(4, 8, 4096, 128, M.F16)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MhaError, match="WORKSPACE"):
        M.decode(q, k, k, workspace=small)
    # a reused workspace with stale contents gives the same result
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    a, la = M.decode(q, k, k, workspace=ws)
    b, lb = M.decode(q, k, k, workspace=ws)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_decode_workload_full_size():
    """The decode workload at its full size, in the launch configuration the
    benchmark times: every head against the oracle, one batch entry at a time."""
    w = W.decode_config()
    got, glse, flags = _run(w)
    assert flags == 0
    q3 = _q3(w)
    for b in range(w.B):
        q = W.to_f64(q3[b:b + 1], w.dtype)
        k = W.to_f64(w.k[b:b + 1], w.dtype)
        v = W.to_f64(w.v[b:b + 1], w.dtype)
        ref, rlse, rflags = oracle.decode(q, k, v, w.lens[b:b + 1], w.scale)
        assert rflags == 0
        assert_parity(got[b:b + 1], ref, w.dtype, f"decode-workload-b{b}")
        assert np.all(np.abs(glse[b:b + 1] - rlse) <= lse_tol(rlse)), b
    assert np.isfinite(got).all() and np.isfinite(glse).all()


def test_decode_very_long_cache():
    """A 65536-key cache: 1024 splits per head, so the merge walks 16 groups
    of 64 splits; lengths cover one split, a group boundary and the full cache."""
    import masked_head_attention_amd as M

    B, H, Lk, D = 3, 2, 65536, 128
    need = M.decode_workspace_size(B, H, Lk, D, M.BF16)
    assert need // (B * H * (D + 2) * 4) == Lk // 64
    w = _work("bf16", B, H, Lk, D, seed=60, lens_range=(1, Lk))
    lens = np.array([37, 64 * 64 + 5, Lk], np.int32)
    _check(w, "decode-long-cache", lens=lens)
