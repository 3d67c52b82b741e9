"""The allocation-free decode entry point (mha_decode_fwd_noalloc) against
the allocating one (mha_decode_fwd), through the C ABI: two calls in a row on
the GPU's one static scratch array, the second with a smaller input. (The
scratch limit is a host-side check, covered without a GPU in test_abi.py.)"""
import pytest

import workloads as W
from helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_head_attention_amd as M

    M.init()  # flag word and the scratch array's device address, once per device


def _pair(w):
    """(noalloc out, lse), (workspace out, lse) for decode workload w."""
    import torch
    import masked_head_attention_amd as M

    q = to_dev(w.q.reshape(w.B, w.H, w.D), w.dtype)
    k, v, lens = to_dev(w.k, w.dtype), to_dev(w.v, w.dtype), to_dev(w.lens, w.dtype)
    need = M.decode_workspace_size(w.B, w.H, w.Lk, w.D, {"f32": 0, "f16": 1, "bf16": 2}[w.dtype])
    assert 0 < need <= M.noalloc_scratch_bytes(), need  # the split plan uses the scratch
    out_a = torch.full_like(q, float("nan"))
    lse_a = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    M.get_flags(clear=True)
    M.decode_noalloc(q, k, v, lens, scale=w.scale, out=out_a, lse=lse_a)
    flags_a = M.get_flags(clear=True)
    out_b, lse_b = M.decode(q, k, v, lens, scale=w.scale)
    flags_b = M.get_flags(clear=True)
    assert flags_a == flags_b
    return (out_a, lse_a), (out_b, lse_b)


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch

    big = W.make("noalloc-big", "f16", B=6, H=8, Lq=1, Lk=3000, D=128, kind=W.PADDING, seed=41,
                 lens_range=(0, 3000))
    small = W.make("noalloc-small", "bf16", B=2, H=3, Lq=1, Lk=900, D=64, kind=W.PADDING,
                   seed=42, lens_range=(1, 900))
    for w in (big, small):  # the second call is smaller: stale partials must not leak in
        print(f"[noalloc] {w.name} {w.dtype} B{w.B} H{w.H} Lk{w.Lk} D{w.D}", flush=True)
        (oa, la), (ob, lb) = _pair(w)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), w.name
        assert torch.equal(la.isnan(), lb.isnan())
        assert torch.equal(la[~la.isnan()], lb[~lb.isnan()]), w.name
        assert not oa.isnan().any()
