"""Pins for the oracle's decode call: one query row per (batch, head) against
a key/value cache with per-sequence lengths (the llama.cpp embedding of
"masked multi head attention" CUDA notes, section 6.1), and the log-sum-exp
of the row's scaled scores (the normaliser of the online softmax in "Why
attention must compute the max first", section 2.4). The log-sum-exp is
checked against scipy's routine, a pure-Python brute force, closed forms and
the exact merge identity of two key ranges that the split kernel relies on."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def _cache(rng, B, H, Lk, D):
    return (rng.normal(0, 1, (B, H, D)), rng.normal(0, 1, (B, H, Lk, D)),
            rng.normal(0, 1, (B, H, Lk, D)))


def test_lse_against_scipy_and_weights_sum_to_one():
    rng = np.random.default_rng(11)
    B, H, Lk, D = 3, 2, 37, 16
    q, k, v = _cache(rng, B, H, Lk, D)
    lens = np.array([37, 5, 20], np.int32)
    scale = 0.3
    out, lse, flags = oracle.decode(q, k, v, lens, scale=scale)
    assert flags == 0
    for b in range(B):
        for h in range(H):
            n = lens[b]
            s = scale * (k[b, h, :n] @ q[b, h])
            assert lse[b, h] == pytest.approx(logsumexp(s), rel=1e-13, abs=1e-13)
            w = np.exp(s - lse[b, h])
            assert w.sum() == pytest.approx(1.0, rel=1e-13)
            np.testing.assert_allclose(out[b, h], w @ v[b, h, :n], rtol=1e-12, atol=1e-13)


def test_brute_force_tiny():
    rng = np.random.default_rng(12)
    B, H, Lk, D = 2, 2, 5, 3
    q, k, v = _cache(rng, B, H, Lk, D)
    lens = np.array([5, 3], np.int32)
    out, lse, _ = oracle.decode(q, k, v, lens, scale=1.25)
    for b in range(B):
        for h in range(H):
            s = [1.25 * math.fsum(q[b, h, d] * k[b, h, j, d] for d in range(D))
                 for j in range(lens[b])]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            assert lse[b, h] == pytest.approx(m + math.log(z), rel=1e-14, abs=1e-14)
            for d in range(D):
                ref = math.fsum(math.exp(s[j] - m) / z * v[b, h, j, d] for j in range(len(s)))
                assert out[b, h, d] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_uniform_keys_closed_form():
    """Equal keys: equal weights, so the output is the mean of the legal
    values and the log-sum-exp is s + ln(n)."""
    rng = np.random.default_rng(13)
    B, H, Lk, D = 2, 3, 50, 8
    q = rng.normal(0, 1, (B, H, D))
    krow = rng.normal(0, 1, (B, H, 1, D))
    k = np.repeat(krow, Lk, axis=2)
    v = rng.normal(0, 1, (B, H, Lk, D))
    lens = np.array([50, 17], np.int32)
    out, lse, _ = oracle.decode(q, k, v, lens, scale=0.5)
    for b in range(B):
        n = lens[b]
        for h in range(H):
            s = 0.5 * float(q[b, h] @ krow[b, h, 0])
            assert lse[b, h] == pytest.approx(s + math.log(n), rel=1e-13, abs=1e-13)
            np.testing.assert_allclose(out[b, h], v[b, h, :n].mean(axis=0), rtol=1e-12,
                                       atol=1e-13)


def test_two_range_merge_identity():
    """The exact merge of two disjoint key ranges: lse = logaddexp(lse1, lse2)
    and out = e^(lse1-lse) out1 + e^(lse2-lse) out2 (ranges via lengths and
    a shifted cache)."""
    rng = np.random.default_rng(14)
    B, H, Lk, D = 2, 2, 40, 8
    q, k, v = _cache(rng, B, H, Lk, D)
    cut = 23
    full, lse, _ = oracle.decode(q, k, v, scale=0.4)
    o1, l1, _ = oracle.decode(q, k[:, :, :cut], v[:, :, :cut], scale=0.4)
    o2, l2, _ = oracle.decode(q, k[:, :, cut:], v[:, :, cut:], scale=0.4)
    np.testing.assert_allclose(lse, np.logaddexp(l1, l2), rtol=1e-13, atol=1e-13)
    merged = np.exp(l1 - lse)[..., None] * o1 + np.exp(l2 - lse)[..., None] * o2
    np.testing.assert_allclose(full, merged, rtol=1e-12, atol=1e-13)


def test_equals_attention_at_one_query_row():
    """Decode is attention with Lq = 1 and the key-padding mask."""
    rng = np.random.default_rng(15)
    B, H, Lk, D = 2, 3, 29, 16
    q, k, v = _cache(rng, B, H, Lk, D)
    lens = np.array([29, 11], np.int32)
    out, _, f1 = oracle.decode(q, k, v, lens)
    ref, f2 = oracle.mha_fwd(q[:, :, None], k, v, oracle.PADDING, lens=lens)
    assert np.array_equal(out, ref[:, :, 0]) and f1 == f2


def test_empty_and_bad_lengths():
    rng = np.random.default_rng(16)
    B, H, Lk, D = 3, 2, 9, 4
    q, k, v = _cache(rng, B, H, Lk, D)
    out, lse, flags = oracle.decode(q, k, v, np.array([0, 9, 4], np.int32))
    assert flags == oracle.FLAG_FULLY_MASKED_ROW
    assert np.all(out[0] == 0.0) and np.all(lse[0] == -np.inf) and np.all(np.isfinite(lse[1:]))
    # lengths beyond [0, Lk] act clamped and raise the length flag
    o2, l2, f2 = oracle.decode(q, k, v, np.array([-3, 12, 4], np.int32))
    assert f2 == oracle.FLAG_FULLY_MASKED_ROW | oracle.FLAG_BAD_LENGTH
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)
    # no keys at all
    o3, l3, f3 = oracle.decode(q, k[:, :, :0], v[:, :, :0])
    assert f3 == oracle.FLAG_FULLY_MASKED_ROW and np.all(o3 == 0) and np.all(l3 == -np.inf)
