"""HIP graph capture of the calls the benchmark times as graphs: the decode
call (split and merge kernels), the backward (dq and dkv kernels) and the
bfloat16 pre-LN call with a workspace (copy kernel and two attention kernels). Each
graph is replayed several times, with eager work and synchronisations in
between, and every replay must reproduce the eager result bit for bit (the
calls enqueue only kernels: no memset or allocation inside the captured
region)."""
import numpy as np
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

    M.init()
    M.get_flags(clear=True)
    yield


def _replays(step, outs, n=4):
    import torch

    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(n):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), f"replay {r} differs"


def test_decode_graph_replays():
    import masked_head_attention_amd as M
    import torch

    w = W.make("graph-decode", "f16", 4, 8, 1, 3000, 128, kind=W.PADDING, seed=50,
               lens_range=(1, 3000))
    q = to_dev(w.q.reshape(w.B, w.H, w.D), w.dtype)
    k, v, lens = to_dev(w.k, w.dtype), to_dev(w.v, w.dtype), to_dev(w.lens, w.dtype)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, M.decode_workspace_size(w.B, w.H, w.Lk, w.D, M.F16)),
                     dtype=torch.uint8, device="cuda")
    _replays(lambda: M.decode(q, k, v, lens, scale=w.scale, out=out, lse=lse, workspace=ws),
             [out, lse])
    assert M.get_flags(clear=True) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_graph_replays(dtype):
    import masked_head_attention_amd as M
    import torch

    w = W.make("graph-bwd", dtype, 1, 4, 200, 200, 64, kind=W.CAUSAL, seed=51)
    q, k, v = (to_dev(getattr(w, n), w.dtype) for n in ("q", "k", "v"))
    g = to_dev(W.grad_output(w), w.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = M.BF16 if dtype == "bf16" else M.F32
    ws = torch.empty(M.bwd_workspace_size(w.B, w.H, w.Lq, code), dtype=torch.uint8,
                     device="cuda")
    _replays(lambda: M.bwd(q, k, v, g, kind=w.kind, scale=w.scale, dq=dq, dk=dk, dv=dv,
                           workspace=ws), [dq, dk, dv])
    assert M.get_flags(clear=True) == 0


def test_prenorm_workspace_graph_replays():
    """Both attention launches serve heads (one head holds a value beyond
    float16's range); the workspace is zeroed between replays, so every replay
    must rewrite the copies and the flags it reads."""
    import masked_head_attention_amd as M
    import torch

    w = W.make("graph-prenorm-ws", "bf16", 2, 4, 150, 300, 64, seed=52, prenorm=True,
               x_mean=0.5, x_std=3.0, residual=True)
    v = W.bf16_bits_to_f32(w.v).astype(np.float64)
    v[1, 2, 77, 5] = 1.0e5
    w.v = W.round_to(v, "bf16")
    x, k, v2, gm, bt = (to_dev(getattr(w, n), w.dtype) for n in ("x", "k", "v", "gamma", "beta"))
    out = torch.empty_like(x)
    # zeros: the alignment padding between the workspace's parts is never
    # written, and the replays below compare the whole buffer
    ws = torch.zeros(M.prenorm_cross_workspace_size(w.B, w.H, w.Lq, w.Lk, w.D, M.BF16),
                     dtype=torch.uint8, device="cuda")
    _replays(lambda: M.prenorm_cross_fwd(x, k, v2, gm, bt, w.eps, residual=x, scale=w.scale,
                                         out=out, workspace=ws), [out, ws])
    assert M.get_flags(clear=True) == 0
