"""Pins for the fp64 oracle: checks against things other than the oracle itself.

* brute force in 40-digit decimal arithmetic with no max subtraction (a
  different algorithm and precision) on tiny inputs, including every keep
  pattern of a 3x3 additive mask;
* a library special case: torch's fp64 scaled_dot_product_attention and
  layer_norm on config-shaped inputs;
* closed forms and invariants: softmax rows sum to 1, causal row 0 is V[0],
  equal scores give prefix means, shift invariance, the two-key logistic form
  at +-88 logits, fully masked rows, mask-kind equivalences, tile counts;
* the numbers the pages print (tests/golden/page_facts.json).
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
CAUSAL, PADDING, ADDITIVE = oracle.CAUSAL, oracle.PADDING, oracle.ADDITIVE


# --------------------------------------------------------------------------
# brute force: direct exp ratio in 40-digit decimals, no max subtraction
# --------------------------------------------------------------------------
def _brute(q, k, v, kind, lens, add, scale):
    getcontext().prec = 40
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    out = np.zeros((B, H, Lq, D))
    full = np.zeros((B, H, Lq), bool)
    for b, h, i in itertools.product(range(B), range(H), range(Lq)):
        num = [Decimal(0)] * D
        den = Decimal(0)
        for j in range(Lk):
            a = add[b, 0, i, j] if kind & ADDITIVE else 0.0
            if (kind & CAUSAL) and j > i:
                continue
            if (kind & PADDING) and j >= lens[b]:
                continue
            if (kind & ADDITIVE) and a == -math.inf:
                continue
            z = Decimal(scale) * sum(Decimal(float(q[b, h, i, d])) * Decimal(float(k[b, h, j, d]))
                                     for d in range(D)) + Decimal(float(a))
            e = z.exp()
            den += e
            for d in range(D):
                num[d] += e * Decimal(float(v[b, h, j, d]))
        if den == 0:
            full[b, h, i] = True
            continue
        for d in range(D):
            out[b, h, i, d] = float(num[d] / den)
    return out, full


def _tiny(rng, B, H, Lq, Lk, D, kind, add_vals=(0.0, 0.75, -1.5, -math.inf)):
    q = rng.standard_normal((B, H, Lq, D))
    k = rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    lens = rng.integers(0, Lk + 1, size=B).astype(np.int32)
    add = rng.choice(np.array(add_vals), size=(B, 1, Lq, Lk))
    return q, k, v, lens, add


@pytest.mark.parametrize("kind", [0, CAUSAL, PADDING, ADDITIVE, CAUSAL | PADDING,
                                  CAUSAL | ADDITIVE])
def test_brute_force_decimal(kind):
    rng = np.random.default_rng(100 + kind)
    for Lq, Lk, D in [(1, 1, 1), (3, 4, 2), (4, 3, 3), (4, 4, 4)]:
        q, k, v, lens, add = _tiny(rng, 2, 2, Lq, Lk, D, kind)
        scale = 0.7
        ref, full = _brute(q, k, v, kind, lens, add, scale)
        out, flags = oracle.mha_fwd(q, k, v, kind, lens, add, scale)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
        assert np.all(out[full] == 0.0)
        assert bool(flags & oracle.FLAG_FULLY_MASKED_ROW) == bool(full.any())


def test_every_keep_pattern_l3():
    """All 2^9 keep/mask patterns of a 3x3 additive mask, kept entries carrying
    finite additive values; fully masked rows give zeros and the flag."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 3, 2))
    k = rng.standard_normal((1, 1, 3, 2))
    v = rng.standard_normal((1, 1, 3, 2))
    vals = rng.standard_normal((1, 1, 3, 3))
    for bits in range(512):
        keep = np.array([(bits >> t) & 1 for t in range(9)], bool).reshape(1, 1, 3, 3)
        add = np.where(keep, vals, -np.inf)
        ref, full = _brute(q, k, v, ADDITIVE, None, add, 0.5)
        out, flags = oracle.mha_fwd(q, k, v, ADDITIVE, None, add, 0.5)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        assert (flags & oracle.FLAG_FULLY_MASKED_ROW != 0) == bool(full.any())
        assert np.array_equal(full[0, 0], ~keep[0, 0].any(axis=1))


# --------------------------------------------------------------------------
# library special case: torch fp64 SDPA and layer_norm
# --------------------------------------------------------------------------
def _torch():
    return pytest.importorskip("torch")


def _decisions_to_additive(w, dec):
    add = np.where(dec.astype(bool), -np.inf, 0.0)[:, None, :, :]
    if w.kind & ADDITIVE:
        a64 = w.f64("add")
        add = np.where(dec[:, None].astype(bool), -np.inf, a64)
    return add


SMALL = {
    1: dict(),
    2: dict(B=2, H=3, Lq=100, Lk=100, lens_range=(40, 100)),
    3: dict(H=2, Lq=150, Lk=150),
    5: dict(B=3, H=2, Lq=160, Lk=160, lens_range=(30, 160), block_p=0.3),
}


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_torch_sdpa_fp64(cfg):
    torch = _torch()
    w = W.config(cfg, **SMALL[cfg])
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    out, flags = oracle.mha_fwd(q, k, v, w.kind, w.lens, w.f64("add"), w.scale)
    dec = oracle.mask_decisions(w.kind, w.B, w.Lq, w.Lk, w.lens, w.f64("add"))
    add = _decisions_to_additive(w, dec)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(add), scale=w.scale).numpy()
    ok = ~dec.all(axis=2)  # rows with a legal key [B, Lq]
    ok = np.broadcast_to(ok[:, None, :], out.shape[:3])
    np.testing.assert_allclose(out[ok], ref[ok], rtol=1e-10, atol=1e-12)
    assert np.all(out[~ok] == 0.0)
    assert bool(flags & oracle.FLAG_FULLY_MASKED_ROW) == bool((~ok).any())


def test_prenorm_vs_torch():
    torch = _torch()
    w = W.config(4, B=2, H=4, Lq=70, Lk=90)
    x, k, v = w.f64("x"), w.f64("k"), w.f64("v")
    g, bt = w.f64("gamma"), w.f64("beta")
    out, flags = oracle.prenorm_cross_fwd(x, k, v, g, bt, w.eps, residual=x)
    tx = torch.from_numpy(x)
    y = torch.nn.functional.layer_norm(tx, (w.H * w.D,), torch.from_numpy(g),
                                       torch.from_numpy(bt), w.eps)
    qh = y.reshape(w.B, w.Lq, w.H, w.D).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qh, torch.from_numpy(k),
                                                         torch.from_numpy(v), scale=w.scale)
    ref = (o.permute(0, 2, 1, 3).reshape(w.B, w.Lq, w.H * w.D) + tx).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-11)
    assert flags == 0
    # the sampled-row entry agrees with the full one
    rows = np.array([[0, 0, 0], [1, 69, 3], [0, 33, 2]])
    r, _ = oracle.prenorm_rows(x, k, v, g, bt, w.eps, rows, residual=x)
    for n, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(r[n], out[b, i, h * w.D:(h + 1) * w.D])


def test_layernorm_vs_torch_and_moments():
    torch = _torch()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7, 96)) * 3 + 0.5
    g = rng.uniform(0.5, 1.5, 96)
    b = rng.standard_normal(96) * 0.1
    y = oracle.layernorm(x, g, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                         torch.from_numpy(b), 1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # with gamma = 1, beta = 0 every token has mean 0 and variance var/(var+eps)
    y1 = oracle.layernorm(x, np.ones(96), np.zeros(96), 1e-5)
    var = x.var(axis=-1)
    np.testing.assert_allclose(y1.mean(axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(y1.var(axis=-1), var / (var + 1e-5), rtol=1e-12)
    # a constant token normalises to 0, so the output is beta
    yc = oracle.layernorm(np.full((1, 96), 2.5), g, b, 1e-5)
    np.testing.assert_allclose(yc[0], b, atol=0)


def test_prenorm_constant_row_gives_mean_v_plus_residual():
    rng = np.random.default_rng(5)
    B, H, Lq, Lk, D = 1, 2, 3, 5, 4
    x = np.full((B, Lq, H * D), 1.25)
    k = rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    out, _ = oracle.prenorm_cross_fwd(x, k, v, np.ones(H * D), np.zeros(H * D), 1e-5,
                                      residual=x)
    mean_v = v.mean(axis=2)  # [B,H,D]
    for h in range(H):
        np.testing.assert_allclose(out[0, :, h * D:(h + 1) * D],
                                   np.broadcast_to(mean_v[0, h] + 1.25, (Lq, D)),
                                   rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------
def test_softmax_rows_sum_to_one():
    w = W.config(5, B=2, H=2, Lq=96, Lk=96, lens_range=(20, 96), block_p=0.3)
    q, k, a = w.f64("q"), w.f64("k"), w.f64("add")
    dec = oracle.mask_decisions(w.kind, w.B, w.Lq, w.Lk, w.lens, a)
    for b, h, i in [(0, 0, 0), (0, 1, 50), (1, 0, 95), (1, 1, 17)]:
        p, f = oracle.probs_row(q, k, b, h, i, w.kind, w.lens, a, w.scale)
        if dec[b, i].all():
            assert np.all(p == 0) and f & oracle.FLAG_FULLY_MASKED_ROW
            continue
        assert abs(math.fsum(p) - 1.0) < 1e-14
        assert np.all(p[dec[b, i].astype(bool)] == 0.0)
        assert np.all(p[~dec[b, i].astype(bool)] > 0.0)


def test_causal_row0_is_v0_and_q0_gives_prefix_means():
    w = W.config(1)
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    out, _ = oracle.mha_fwd(q, k, v, CAUSAL, scale=w.scale)
    assert np.array_equal(out[:, :, 0, :], v[:, :, 0, :])
    out0, _ = oracle.mha_fwd(np.zeros_like(q), k, v, CAUSAL, scale=w.scale)
    prefix = np.cumsum(v, axis=2) / np.arange(1, w.Lk + 1)[None, None, :, None]
    np.testing.assert_allclose(out0, prefix, rtol=1e-13, atol=1e-14)


def test_q0_causal_padding_means():
    rng = np.random.default_rng(11)
    B, H, L, D = 3, 2, 20, 4
    k = rng.standard_normal((B, H, L, D))
    v = rng.standard_normal((B, H, L, D))
    lens = np.array([5, 20, 1], np.int32)
    out, f = oracle.mha_fwd(np.zeros((B, H, L, D)), k, v, CAUSAL | PADDING, lens)
    assert f == 0
    for b in range(B):
        for i in range(L):
            n = min(i, lens[b] - 1) + 1
            np.testing.assert_allclose(out[b, :, i], v[b, :, :n].mean(axis=1), rtol=1e-13,
                                       atol=1e-14)


def test_shift_invariance():
    w = W.config(5, B=2, H=2, Lq=64, Lk=64, lens_range=(20, 64), block_p=0.2)
    q, k, v, a = w.f64("q"), w.f64("k"), w.f64("v"), w.f64("add")
    out, _ = oracle.mha_fwd(q, k, v, w.kind, None, a, w.scale)
    a2 = a.copy()
    shift = np.random.default_rng(1).uniform(-30, 30, size=(w.B, 1, w.Lq, 1))
    a2 = np.where(np.isfinite(a2), a2 + shift, a2)
    out2, _ = oracle.mha_fwd(q, k, v, w.kind, None, a2, w.scale)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("z", [88.0, -88.0, 11.0])
def test_two_key_logistic_at_large_logits(z):
    # D=1, scale 1: logits are z*1 and z*(-1) -> weights sigma(2z), 1 - sigma(2z)
    q = np.array([[[[z]]]])
    k = np.array([[[[1.0], [-1.0]]]])
    v = np.array([[[[3.0], [-2.0]]]])
    out, f = oracle.mha_fwd(q, k, v, 0, scale=1.0)
    sig = 1.0 / (1.0 + math.exp(-2 * z)) if z > -300 else 0.0
    assert f == 0 and np.isfinite(out).all()
    assert abs(out[0, 0, 0, 0] - (sig * 3.0 + (1 - sig) * -2.0)) < 1e-13


def test_fully_masked_row_and_flags():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 1, 4, 3))
    k = rng.standard_normal((2, 1, 4, 3))
    v = rng.standard_normal((2, 1, 4, 3))
    lens = np.array([0, 4], np.int32)
    out, f = oracle.mha_fwd(q, k, v, PADDING, lens)
    assert np.all(out[0] == 0.0) and f == oracle.FLAG_FULLY_MASKED_ROW
    assert oracle.fully_masked_rows(PADDING, 2, 1, 4, 4, lens) == 4
    out, f = oracle.mha_fwd(q, k, v, PADDING, np.array([-1, 9], np.int32))
    assert f == oracle.FLAG_FULLY_MASKED_ROW | oracle.FLAG_BAD_LENGTH
    out, f = oracle.mha_fwd(q, k, v, PADDING, np.array([9, 4], np.int32))
    assert f == oracle.FLAG_BAD_LENGTH
    vn = v.copy()
    vn[1, 0, 2, 1] = np.nan
    out, f = oracle.mha_fwd(q, k, vn, 0)
    assert f & oracle.FLAG_NONFINITE and np.isnan(out[1, 0, :, 1]).all()


def test_kind_equivalences_bitwise():
    rng = np.random.default_rng(9)
    B, H, L, D = 3, 2, 37, 8
    q, k, v = (rng.standard_normal((B, H, L, D)) for _ in range(3))
    lens = np.array([1, 20, 37], np.int32)
    pad, _ = oracle.mha_fwd(q, k, v, PADDING, lens)
    add = np.zeros((B, 1, L, L))
    for b in range(B):
        add[b, 0, :, lens[b]:] = -np.inf
    addp, _ = oracle.mha_fwd(q, k, v, ADDITIVE, None, add)
    assert np.array_equal(pad, addp)
    cau, _ = oracle.mha_fwd(q, k, v, CAUSAL)
    addc = np.broadcast_to(np.triu(np.full((L, L), -np.inf), 1), (B, 1, L, L))
    addc_out, _ = oracle.mha_fwd(q, k, v, ADDITIVE, None, np.where(np.isinf(addc), -np.inf, 0.0))
    assert np.array_equal(cau, addc_out)


def test_mask_probe_reads_back_decisions():
    """Q = 0 and V one-hot in key block r: out[i, d] = legal(i, r*D + d) / n_i,
    so the output spells the mask bitmap."""
    w = W.config(5, B=2, H=1, Lq=64, Lk=64, lens_range=(10, 64), block_p=0.3, block=16)
    a = w.f64("add")
    dec = oracle.mask_decisions(w.kind, w.B, w.Lq, w.Lk, None, a).astype(bool)
    D = 16
    n = (~dec).sum(axis=2)
    for r in range(w.Lk // D):
        v = np.zeros((w.B, 1, w.Lk, D))
        for d in range(D):
            v[:, 0, r * D + d, d] = 1.0
        out, _ = oracle.mha_fwd(np.zeros((w.B, 1, w.Lq, D)), np.zeros((w.B, 1, w.Lk, D)), v,
                                w.kind, None, a)
        legal = ~dec[:, :, r * D:(r + 1) * D]
        expect = np.where(n[:, :, None] > 0, legal / np.maximum(n, 1)[:, :, None], 0.0)
        np.testing.assert_allclose(out[:, 0], expect, rtol=1e-14, atol=1e-15)


def test_unmasked_pairs_closed_forms():
    L = 100
    assert oracle.unmasked_pairs(CAUSAL, 2, 3, L, L) == 2 * 3 * L * (L + 1) // 2
    lens = np.array([10, 50], np.int32)
    assert oracle.unmasked_pairs(PADDING, 2, 3, L, L, lens) == 3 * L * (10 + 50)
    cp = sum(sum(min(i, lb - 1) + 1 for i in range(L)) for lb in lens)
    assert oracle.unmasked_pairs(CAUSAL | PADDING, 2, 3, L, L, lens) == 3 * cp


@pytest.mark.parametrize("L,t", [(128, 16), (2048, 64), (96, 32), (100, 32)])
def test_causal_tile_counts_closed_form(L, t):
    T = -(-L // t)
    comp, skip = oracle.tile_counts(CAUSAL, 1, 2, L, L, t, t)
    assert comp == 2 * T * (T + 1) // 2 and comp + skip == 2 * T * T


def test_tile_counts_padding_rect():
    lens = np.array([33, 64, 0], np.int32)
    comp, skip = oracle.tile_counts(PADDING, 3, 1, 64, 64, 32, 16, lens)
    # rows: 2 blocks; key blocks of 16: len 33 -> 3 blocks, 64 -> 4, 0 -> 0
    assert comp == 2 * (3 + 4 + 0) and skip == 2 * (1 + 0 + 4)


# --------------------------------------------------------------------------
# numbers printed on the pages
# --------------------------------------------------------------------------
def _facts():
    with open(os.path.join(HERE, "golden", "page_facts.json")) as f:
        return json.load(f)


def test_page_causal_skip_fraction():
    f = _facts()["causal_skip_fraction_l128"]
    t = f["tile"]
    comp, skip = oracle.tile_counts(CAUSAL, 1, 1, f["seq_len"], f["seq_len"], t[0], t[1])
    frac = skip / (comp + skip)
    assert abs(frac - f["value"]) <= f["approx_tolerance"]
    assert frac == 28 / 64


def test_page_shape_and_overflow_facts():
    f = _facts()
    s = f["qkt_elements_b4_h8_l128"]
    assert int(np.prod(s["shape"])) == s["value"]
    assert f["mask_bytes_l128"]["value"] == f["mask_bytes_l128"]["seq_len"] ** 2
    # the fp16 / fp32 overflow points that motivate subtracting the max
    e = f["fp16_exp_overflow"]
    with np.errstate(over="ignore"):
        assert np.float16(math.exp(10)) > e["exp10_exceeds"]
        assert np.isinf(np.float16(math.exp(e["overflow_at"])))
        assert float(np.finfo(np.float16).max) == e["fp16_max"]
        assert np.isinf(np.exp(np.float32(f["fp32_exp_overflow_logit"]["value"] + 1)))
    assert f["fp16_min_as_mask_value"]["value"] == float(np.finfo(np.float16).min)
    # with the max subtracted the oracle stays finite at those logits
    for z in (f["fp32_exp_overflow_logit"]["value"], e["overflow_at"]):
        q = np.full((1, 1, 1, 1), float(z))
        out, fl = oracle.mha_fwd(q, np.ones((1, 1, 3, 1)), np.ones((1, 1, 3, 1)), 0, scale=1.0)
        assert fl == 0 and abs(out[0, 0, 0, 0] - 1.0) < 1e-15


def test_fp16_min_mask_is_a_finite_bias_not_a_mask():
    """-65504 as a mask value is a large finite bias: a row masked only with it
    gets uniform weights over those keys, not zeros."""
    q = np.zeros((1, 1, 1, 2))
    k = np.zeros((1, 1, 3, 2))
    v = np.array([[[[1.0, 0.0], [2.0, 0.0], [6.0, 0.0]]]])
    add = np.full((1, 1, 1, 3), -65504.0)
    out, f = oracle.mha_fwd(q, k, v, ADDITIVE, None, add)
    assert f == 0 and abs(out[0, 0, 0, 0] - 3.0) < 1e-13
