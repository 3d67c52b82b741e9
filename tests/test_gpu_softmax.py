"""GPU parity of the row softmax over a materialised score tensor (the
row-softmax workload of "Why attention must compute the max first", section
2.1) against the fp64 oracle, through the C ABI.

Bar: |gpu - oracle| <= tol + half an output ulp elementwise (tol 1e-5 for
float32, 2e-3 for float16/bfloat16); flags agree exactly.
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


def _run(w, out_same=False):
    import masked_head_attention_amd as M

    s = to_dev(w.s, w.dtype)
    print(f"[softmax] {w.name} {w.dtype} shape {w.shape} scale {w.scale} seed {w.seed}",
          flush=True)
    out = M.softmax_rows(s, out=s if out_same else None, scale=w.scale)
    flags = M.get_flags(clear=True)
    return from_dev(out), flags


def _check(w, what, out_same=False):
    got, flags = _run(w, out_same)
    ref, rflags = oracle.softmax_rows(w.f64(), w.scale)
    assert_parity(got, ref, w.dtype, what)
    assert flags == rflags, (what, flags, rflags)


# register path (16-byte rows of up to 4096 16-bit / 2048 float32 values) and
# the general two-pass path (longer or unaligned rows)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [1, 7, 8, 64, 520, 1001, 2048, 4096, 5000])
def test_rows_parity(dtype, cols):
    w = W.make_scores("rows", dtype, (3, 37, cols), seed=cols, std=3.0, masked_p=0.1,
                      masked_rows=2 if cols > 1 else 0)
    _check(w, f"softmax-{dtype}-{cols}")


@pytest.mark.parametrize("scale", [0.0, 0.125, 4.0])
def test_scales(scale):
    w = W.make_scores("scaled", "f16", (50, 2048), seed=3, std=2.0, masked_p=0.05, scale=scale)
    _check(w, f"softmax-scale-{scale}")


def test_large_logits_stay_finite():
    # scores far beyond exp's range: the row maximum is subtracted first
    w = W.make_scores("large", "f32", (20, 300), seed=4, std=300.0)
    _check(w, "softmax-large-logits")


def test_in_place():
    w = W.make_scores("inplace", "bf16", (64, 2048), seed=5, masked_p=0.2, masked_rows=3)
    _check(w, "softmax-in-place", out_same=True)
    w = W.make_scores("inplace-gen", "f16", (16, 3001), seed=6, masked_p=0.2)
    _check(w, "softmax-in-place-general", out_same=True)


def test_fully_masked_and_nan_flags():
    import masked_head_attention_amd as M
    import torch

    s = torch.zeros(4, 2048, dtype=torch.float16, device="cuda")
    s[1] = float("-inf")
    out = M.softmax_rows(s)
    assert M.get_flags(clear=True) == M.FLAG_FULLY_MASKED_ROW
    o = out.float().cpu().numpy()
    assert np.all(o[1] == 0.0) and np.allclose(o[0], 1.0 / 2048)
    s[2, 5] = float("nan")
    M.softmax_rows(s, out=out)
    assert M.get_flags(clear=True) == M.FLAG_FULLY_MASKED_ROW | M.FLAG_NONFINITE


def test_empty_calls():
    import masked_head_attention_amd as M
    import torch

    for shape in [(0, 16), (4, 0)]:
        s = torch.zeros(shape, dtype=torch.float16, device="cuda")
        M.softmax_rows(s)
    assert M.get_flags(clear=True) == 0


def test_workload_full_size():
    """The pages' 1 x 32 x 2048 x 2048 float16 tensor, as the benchmark runs
    it: every row against the oracle, in blocks of 8192 rows."""
    w = W.softmax_config()
    got, flags = _run(w)
    assert flags == 0
    flat = got.reshape(w.rows, w.cols)
    src = w.f64().reshape(w.rows, w.cols)
    for r0 in range(0, w.rows, 8192):
        ref, rflags = oracle.softmax_rows(src[r0:r0 + 8192], w.scale)
        assert rflags == 0
        assert_parity(flat[r0:r0 + 8192], ref, w.dtype, f"softmax-workload-rows{r0}")
