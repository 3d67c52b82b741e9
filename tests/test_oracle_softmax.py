"""Pins for the oracle's row softmax over a materialised score tensor (the
standalone row-softmax workload of "Why attention must compute the max first",
section 2.1): a brute force in exact-sum pure Python, torch's float64 softmax
as a library special case, closed forms, invariants and the flag cases."""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
NEG = -np.inf


def _brute(row, scale):
    """Independent path: math.exp and math.fsum, masked entries skipped."""
    legal = [scale * float(x) for x in row if x != NEG]
    if not legal:
        return [0.0] * len(row), oracle.FLAG_FULLY_MASKED_ROW
    m = max(legal)
    z = math.fsum(math.exp(v - m) for v in legal)
    return [0.0 if x == NEG else math.exp(scale * float(x) - m) / z for x in row], 0


@pytest.mark.parametrize("scale", [1.0, 0.125, 3.0])
def test_brute_force_small_rows(scale):
    rng = np.random.default_rng(7)
    s = rng.normal(0, 3, (12, 9))
    s[rng.random(s.shape) < 0.25] = NEG
    s[5, :] = NEG  # a fully masked row
    p, flags = oracle.softmax_rows(s, scale)
    want_flags = 0
    for r in range(s.shape[0]):
        ref, f = _brute(s[r], scale)
        want_flags |= f
        np.testing.assert_allclose(p[r], ref, rtol=1e-13, atol=1e-300)
    assert flags == want_flags == oracle.FLAG_FULLY_MASKED_ROW


def test_torch_softmax_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    s = rng.normal(0, 4, (64, 257))
    s[rng.random(s.shape) < 0.1] = NEG
    s[:, 0] = rng.normal(0, 4, 64)  # no row fully masked
    p, flags = oracle.softmax_rows(s, 0.7)
    ref = torch.softmax(torch.from_numpy(s) * 0.7, dim=-1).numpy()
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-15)
    assert flags == 0


@pytest.mark.parametrize("z", [-30.0, -2.0, 0.0, 0.5, 40.0])
def test_two_entry_logistic(z):
    p, _ = oracle.softmax_rows(np.array([[0.0, z]]))
    # softmax([0, z]) = (sigma(-z), sigma(z)), each formed without cancellation
    np.testing.assert_allclose(p[0], [1.0 / (1.0 + math.exp(z)), 1.0 / (1.0 + math.exp(-z))],
                               rtol=1e-14, atol=1e-300)


def test_uniform_and_dominant_rows():
    p, _ = oracle.softmax_rows(np.full((3, 10), 2.5))
    assert np.all(p == 0.1)
    p, _ = oracle.softmax_rows(np.array([[1000.0, 0.0, -5.0]]))  # exp(-1000) underflows
    assert p[0, 0] == 1.0 and p[0, 1] == 0.0 and p[0, 2] == 0.0


def test_rows_sum_to_one_shift_and_scale_invariance():
    rng = np.random.default_rng(11)
    s = rng.normal(0, 5, (40, 100))
    s[rng.random(s.shape) < 0.2] = NEG
    s[:, 3] = 1.0
    p, _ = oracle.softmax_rows(s, 0.5)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)
    shifted = np.where(s == NEG, NEG, s + 17.25)
    p2, _ = oracle.softmax_rows(shifted, 0.5)
    np.testing.assert_allclose(p2, p, rtol=1e-12, atol=1e-300)
    # scaling inside equals pre-scaled scores: bit for bit
    p3, _ = oracle.softmax_rows(np.where(s == NEG, NEG, 0.5 * s), 1.0)
    assert np.array_equal(p3, p)


def test_flags_fully_masked_and_nan():
    p, f = oracle.softmax_rows(np.array([[NEG, NEG], [0.0, 1.0]]))
    assert f == oracle.FLAG_FULLY_MASKED_ROW and np.all(p[0] == 0.0)
    p, f = oracle.softmax_rows(np.array([[0.0, np.nan, 1.0]]))
    assert f & oracle.FLAG_NONFINITE


def test_page_workload_size():
    with open(os.path.join(HERE, "golden", "page_facts.json")) as fh:
        fact = json.load(fh)["row_softmax_workload"]
    assert int(np.prod(fact["shape"])) * 2 == fact["bytes"] == 256 * 2**20
