"""Pins for the oracle's backward (the gradients of the masked attention
forward for an upstream gradient dO, through the softmax Jacobian of "Why
attention must compute the max first", section 3.3). Checked against central
finite differences of the oracle's forward (an independent code path),
torch's fp64 autograd of scaled_dot_product_attention (a library special
case), and closed forms / invariants that a dropped term, a wrong sign or a
transposed operand would break."""
import numpy as np
import pytest

import oracle

C, P, A = oracle.CAUSAL, oracle.PADDING, oracle.ADDITIVE


def _inputs(seed, B=1, H=2, Lq=5, Lk=6, D=3):
    r = np.random.default_rng(seed)
    return [r.normal(size=s) for s in [(B, H, Lq, D), (B, H, Lk, D), (B, H, Lk, D), (B, H, Lq, D)]]


def _loss(q, k, v, g, kind, lens, add, scale):
    out, _ = oracle.mha_fwd(q, k, v, kind, lens, add, scale)
    return float((out * g).sum())


@pytest.mark.parametrize("kind", [0, C, P, C | P, A, C | A])
def test_finite_differences(kind):
    q, k, v, g = _inputs(100 + kind, B=2, Lq=5, Lk=6)
    r = np.random.default_rng(7)
    lens = np.array([6, 3], np.int32) if kind & P else None
    add = None
    if kind & A:
        add = np.where(r.random((2, 1, 5, 6)) < 0.3, -np.inf, r.normal(size=(2, 1, 5, 6)))
    scale = 0.7
    dq, dk, dv, _ = oracle.mha_bwd(q, k, v, g, kind, lens, add, scale)
    h = 1e-6
    for name, x, grad in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fd[idx] = (_loss(**{**args, name: xp}, g=g, kind=kind, lens=lens, add=add, scale=scale)
                       - _loss(**{**args, name: xm}, g=g, kind=kind, lens=lens, add=add,
                               scale=scale)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=f"d{name} kind {kind}")


def test_against_torch_autograd_sdpa():
    torch = pytest.importorskip("torch")
    q, k, v, g = _inputs(3, B=2, H=3, Lq=9, Lk=11, D=8)
    r = np.random.default_rng(9)
    add = np.where(r.random((2, 1, 9, 11)) < 0.25, -np.inf, r.normal(size=(2, 1, 9, 11)))
    add[..., 0] = 0.0  # no fully masked row (torch gives NaN there)
    scale = 0.4
    dq, dk, dv, _ = oracle.mha_bwd(q, k, v, g, A, None, add, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.tensor(add, dtype=torch.float64), scale=scale)
    o.backward(torch.tensor(g, dtype=torch.float64))
    for a, b in [(dq, tq.grad), (dk, tk.grad), (dv, tv.grad)]:
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_key_gradients_sum_to_zero():
    """Every row's dS sums to 0 over its keys (the softmax Jacobian's rows sum
    to 0), so sum_j dK_j = scale sum_i (sum_j dS_ij) q_i = 0 per head."""
    q, k, v, g = _inputs(4, B=2, H=2, Lq=7, Lk=7, D=4)
    for kind, lens in [(0, None), (C, None), (C | P, np.array([7, 4], np.int32))]:
        _, dk, _, _ = oracle.mha_bwd(q, k, v, g, kind, lens)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13)


def test_equal_keys_give_zero_query_gradient():
    q, k, v, g = _inputs(5, Lq=4, Lk=6, D=3)
    k = np.repeat(k[:, :, :1], 6, axis=2)
    dq, _, _, _ = oracle.mha_bwd(q, k, v, g, C)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)


def test_zero_queries_closed_form():
    """Q = 0: uniform weights over the legal keys, so dV_j = sum over the rows
    i that see key j of dO_i / n_i, and dK = scale * dS^T Q = 0 exactly."""
    q, k, v, g = _inputs(6, B=1, H=1, Lq=5, Lk=5, D=3)
    q = np.zeros_like(q)
    _, dk, dv, _ = oracle.mha_bwd(q, k, v, g, C)
    assert np.all(dk == 0.0)
    ref = np.zeros_like(dv)
    for i in range(5):
        for j in range(i + 1):
            ref[0, 0, j] += g[0, 0, i] / (i + 1)
    np.testing.assert_allclose(dv, ref, rtol=1e-14, atol=1e-15)


def test_fully_masked_row_has_no_gradient():
    q, k, v, g = _inputs(7, B=1, H=1, Lq=4, Lk=5, D=3)
    add = np.zeros((1, 1, 4, 5))
    add[0, 0, 2] = -np.inf  # row 2 sees no key
    dq, dk, dv, f = oracle.mha_bwd(q, k, v, g, A, None, add)
    assert f == oracle.FLAG_FULLY_MASKED_ROW and np.all(dq[0, 0, 2] == 0.0)
    g2 = g.copy()
    g2[0, 0, 2] = 1e3  # that row's upstream gradient reaches nothing
    dq2, dk2, dv2, _ = oracle.mha_bwd(q, k, v, g2, A, None, add)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2) and np.array_equal(dq, dq2)


def test_additive_shift_invariance():
    q, k, v, g = _inputs(8, B=1, H=2, Lq=4, Lk=6, D=5)
    r = np.random.default_rng(1)
    add = np.where(r.random((1, 1, 4, 6)) < 0.3, -np.inf, r.normal(size=(1, 1, 4, 6)))
    add[..., 1] = 0.0
    a = oracle.mha_bwd(q, k, v, g, A, None, add)
    b = oracle.mha_bwd(q, k, v, g, A, None, add + np.array([0.5, -3.0, 7.0, 0.0])[:, None])
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_padding_equals_additive():
    q, k, v, g = _inputs(9, B=2, H=1, Lq=4, Lk=6, D=3)
    lens = np.array([6, 2], np.int32)
    add = np.zeros((2, 1, 4, 6))
    add[1, :, :, 2:] = -np.inf
    a = oracle.mha_bwd(q, k, v, g, C | P, lens)
    b = oracle.mha_bwd(q, k, v, g, C | A, None, add)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
