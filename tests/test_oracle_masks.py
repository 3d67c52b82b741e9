"""Pins for the oracle's extra mask forms: the keep-mask (0 masks a key, any
other value keeps it; "masked multi head attention" CUDA notes, section 4.2
kernel) and per-head mask tensors [B,H,Lq,Lk]. Each reduces exactly to a form
already pinned (the additive -inf mask shared by the heads), and a pure-Python
brute force checks the keep-mask on tiny inputs."""
import math

import numpy as np
import pytest

import oracle
from oracle import ADDITIVE, CAUSAL, KEEP, PER_HEAD


def _qkv(rng, B, H, Lq, Lk, D):
    return (rng.normal(0, 1, (B, H, Lq, D)), rng.normal(0, 1, (B, H, Lk, D)),
            rng.normal(0, 1, (B, H, Lk, D)))


def _keep(rng, shape, p_masked=0.3):
    m = rng.uniform(0.5, 2.0, shape)
    m[rng.random(shape) < p_masked] = 0.0
    return m


@pytest.mark.parametrize("extra", [0, CAUSAL])
def test_keep_equals_additive_minus_inf(extra):
    rng = np.random.default_rng(1)
    B, H, Lq, Lk, D = 2, 3, 17, 23, 8
    q, k, v = _qkv(rng, B, H, Lq, Lk, D)
    keep = _keep(rng, (B, 1, Lq, Lk))
    keep[0, 0, 4] = 0.0  # a fully masked row
    add = np.where(keep == 0.0, -np.inf, 0.0)
    o1, f1 = oracle.mha_fwd(q, k, v, KEEP | extra, add=keep)
    o2, f2 = oracle.mha_fwd(q, k, v, ADDITIVE | extra, add=add)
    assert np.array_equal(o1, o2) and f1 == f2 == oracle.FLAG_FULLY_MASKED_ROW
    for fn in (oracle.unmasked_pairs, oracle.fully_masked_rows):
        assert fn(KEEP | extra, B, H, Lq, Lk, add=keep) == fn(ADDITIVE | extra, B, H, Lq, Lk,
                                                              add=add)
    assert oracle.tile_counts(KEEP | extra, B, H, Lq, Lk, 8, 8, add=keep) == \
        oracle.tile_counts(ADDITIVE | extra, B, H, Lq, Lk, 8, 8, add=add)
    assert np.array_equal(oracle.mask_decisions(KEEP | extra, B, Lq, Lk, add=keep),
                          oracle.mask_decisions(ADDITIVE | extra, B, Lq, Lk, add=add))


@pytest.mark.parametrize("kind", [ADDITIVE, KEEP, ADDITIVE | CAUSAL])
def test_per_head_replicated_equals_shared(kind):
    rng = np.random.default_rng(2)
    B, H, Lq, Lk, D = 2, 4, 13, 19, 8
    q, k, v = _qkv(rng, B, H, Lq, Lk, D)
    if kind & KEEP:
        m = _keep(rng, (B, 1, Lq, Lk))
    else:
        m = np.where(rng.random((B, 1, Lq, Lk)) < 0.3, -np.inf, rng.normal(0, 0.5, (B, 1, Lq, Lk)))
    mh = np.repeat(m, H, axis=1)
    o1, f1 = oracle.mha_fwd(q, k, v, kind, add=m)
    o2, f2 = oracle.mha_fwd(q, k, v, kind | PER_HEAD, add=mh)
    assert np.array_equal(o1, o2) and f1 == f2
    assert oracle.unmasked_pairs(kind, B, H, Lq, Lk, add=m) == \
        oracle.unmasked_pairs(kind | PER_HEAD, B, H, Lq, Lk, add=mh)


@pytest.mark.parametrize("kind", [ADDITIVE, KEEP, KEEP | CAUSAL])
def test_per_head_slices(kind):
    """Head h of a per-head call = a one-head call with head h's mask slice."""
    rng = np.random.default_rng(3)
    B, H, Lq, Lk, D = 2, 3, 11, 14, 8
    q, k, v = _qkv(rng, B, H, Lq, Lk, D)
    if kind & KEEP:
        mh = _keep(rng, (B, H, Lq, Lk))
    else:
        mh = np.where(rng.random((B, H, Lq, Lk)) < 0.3, -np.inf,
                      rng.normal(0, 0.5, (B, H, Lq, Lk)))
    out, _ = oracle.mha_fwd(q, k, v, kind | PER_HEAD, add=mh)
    pairs = 0
    for h in range(H):
        sl = slice(h, h + 1)
        oh, _ = oracle.mha_fwd(q[:, sl], k[:, sl], v[:, sl], kind, add=mh[:, sl])
        assert np.array_equal(out[:, sl], oh)
        pairs += oracle.unmasked_pairs(kind, B, 1, Lq, Lk, add=mh[:, sl])
    assert oracle.unmasked_pairs(kind | PER_HEAD, B, H, Lq, Lk, add=mh) == pairs
    dec = oracle.mask_decisions(kind | PER_HEAD, B, Lq, Lk, add=mh, H=H)
    assert dec.shape == (B, H, Lq, Lk)
    for h in range(H):
        assert np.array_equal(dec[:, h], oracle.mask_decisions(kind, B, Lq, Lk,
                                                               add=mh[:, h:h + 1]))


def test_per_head_prenorm_slices():
    rng = np.random.default_rng(4)
    B, H, Lq, Lk, D = 2, 2, 9, 12, 8
    x = rng.normal(0.5, 2.0, (B, Lq, H * D))
    k, v = rng.normal(0, 1, (B, H, Lk, D)), rng.normal(0, 1, (B, H, Lk, D))
    g, be = rng.uniform(0.5, 1.5, H * D), rng.normal(0, 0.1, H * D)
    mh = _keep(rng, (B, H, Lq, Lk))
    out, _ = oracle.prenorm_cross_fwd(x, k, v, g, be, 1e-5, residual=x, kind=KEEP | PER_HEAD,
                                      add=mh)
    m0 = np.repeat(mh[:, :1], H, axis=1)  # head 0's mask for every head
    ref, _ = oracle.prenorm_cross_fwd(x, k, v, g, be, 1e-5, residual=x, kind=KEEP | PER_HEAD,
                                      add=m0)
    assert np.array_equal(out[..., :D], ref[..., :D])  # head 0 unchanged


def test_keep_brute_force_tiny():
    """Pure Python: legal keys are those with a nonzero keep value (and j <= i
    for causal); weights exp(s - max) / sum; keep values are never added."""
    rng = np.random.default_rng(5)
    B, H, L, D = 1, 2, 4, 3
    q, k, v = _qkv(rng, B, H, L, L, D)
    keep = _keep(rng, (B, H, L, L), 0.4)
    scale = 0.7
    for kind in (KEEP | PER_HEAD, KEEP | PER_HEAD | CAUSAL):
        out, _ = oracle.mha_fwd(q, k, v, kind, add=keep, scale=scale)
        for h in range(H):
            for i in range(L):
                legal = [j for j in range(L) if keep[0, h, i, j] != 0.0
                         and not (kind & CAUSAL and j > i)]
                if not legal:
                    assert np.all(out[0, h, i] == 0.0)
                    continue
                s = {j: scale * math.fsum(q[0, h, i, d] * k[0, h, j, d] for d in range(D))
                     for j in legal}
                m = max(s.values())
                z = math.fsum(math.exp(s[j] - m) for j in legal)
                ref = [math.fsum(math.exp(s[j] - m) / z * v[0, h, j, d] for j in legal)
                       for d in range(D)]
                np.testing.assert_allclose(out[0, h, i], ref, rtol=1e-12, atol=1e-14)

