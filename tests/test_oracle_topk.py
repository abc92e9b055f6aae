"""Pins for the top-K cache producer's oracle (CPU).

Each pin fixes the oracle against something other than itself: a hand-worked
example, torch's topk / log_softmax, a pure-Python sort on tiny rows, closed
forms and invariants, and planted mistakes that must each fail a pin.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import synth
from oracle.topk import topk_probs


def test_hand_worked_example():
    # exp(logits) = 1, 2, 3, 0, 2 -> Z = 8; order by logit, the tie (ln 2) by index
    x = np.array([[0.0, math.log(2), math.log(3), -math.inf, math.log(2)]])
    idx, p, lse = topk_probs(x, 5)
    assert idx.tolist() == [[2, 1, 4, 0, 3]]
    assert np.allclose(p, [[3 / 8, 2 / 8, 2 / 8, 1 / 8, 0.0]], rtol=0, atol=1e-15)
    assert lse[0] == pytest.approx(math.log(8), abs=1e-15)


def test_matches_torch_topk_and_log_softmax_on_distinct_values():
    g = np.random.default_rng(3)
    x = g.standard_normal((16, 1000)) * 3.0
    K = 37
    idx, p, lse = topk_probs(x, K)
    t = torch.from_numpy(x)
    vals, ti = torch.topk(t, K, dim=1, largest=True, sorted=True)
    assert np.array_equal(idx, ti.numpy().astype(np.int32))
    ref_p = torch.exp(torch.log_softmax(t, dim=1)).gather(1, ti).numpy()
    assert np.allclose(p, ref_p, rtol=1e-13, atol=0)
    assert np.allclose(lse, torch.logsumexp(t, dim=1).numpy(), rtol=1e-14, atol=0)


def _brute(row, K):
    """Pure-Python selection: sort (value, index) pairs by value down, index up."""
    pairs = sorted(((float(v) + 0.0, i) for i, v in enumerate(row)), key=lambda q: (-q[0], q[1]))
    z = sum(math.exp(v) for v in row if v != -math.inf)
    return [i for _, i in pairs[:K]], [math.exp(v) / z for v, _ in pairs[:K]]


def test_ties_and_signed_zero_against_brute_force():
    rows = [
        [1.0, 2.0, 2.0, 0.0, -0.0, 2.0, -1.0, 0.0],
        [-0.0, 0.0, -0.0, 0.0, 0.0, -0.0, 5.0, -math.inf],
        [3.0] * 8,
    ]
    for row in rows:
        for K in range(1, 9):
            idx, p, _ = topk_probs(np.array([row]), K)
            bi, bp = _brute(row, K)
            assert idx[0].tolist() == bi, (row, K)
            assert np.allclose(p[0], bp, rtol=1e-14, atol=1e-300)


def test_exhaustive_tiny_rows():
    """Every row over a 3-value alphabet of length 5, all K."""
    for row in itertools.product([-1.0, 0.5, 2.0], repeat=5):
        for K in range(1, 6):
            idx, p, _ = topk_probs(np.array([row]), K)
            bi, bp = _brute(row, K)
            assert idx[0].tolist() == bi
            assert np.allclose(p[0], bp, rtol=1e-14)


def test_closed_form_from_known_distribution():
    """Logits log q for a known q give p = q, sorted."""
    q = np.array([0.05, 0.4, 0.1, 0.25, 0.2])
    idx, p, lse = topk_probs(np.log(q)[None, :] + 7.0, 3)   # a shift changes nothing
    assert idx[0].tolist() == [1, 3, 4]
    assert np.allclose(p[0], [0.4, 0.25, 0.2], rtol=1e-14)
    assert lse[0] == pytest.approx(7.0, abs=1e-14)


def test_invariants_on_synthetic_teacher_logits():
    bits = synth.make_teacher_logits(8, 5000, seed=11)
    x = synth.bf16_bits_to_f32(bits)
    idx, p, lse = topk_probs(x, 5000)
    # K = V: a permutation, probabilities sum to one, non-increasing
    for r in range(8):
        assert sorted(idx[r].tolist()) == list(range(5000))
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-12)
    assert np.all(np.diff(p, axis=1) <= 0)
    # top-100 is the prefix of the full order; its mass is below one
    i100, p100, _ = topk_probs(x, 100)
    assert np.array_equal(i100, idx[:, :100]) and np.all(p100.sum(axis=1) < 1)
    # shift invariance of indices and probabilities
    i2, p2, l2 = topk_probs(x.astype(np.float64) + 3.25, 100)
    assert np.array_equal(i2, i100) and np.allclose(p2, p100, rtol=1e-12)
    assert np.allclose(l2, lse + 3.25, rtol=1e-14)


@pytest.mark.parametrize("bad", [math.nan, math.inf])
def test_invalid_logits_rejected(bad):
    x = np.zeros((2, 10))
    x[1, 3] = bad
    with pytest.raises(ValueError):
        topk_probs(x, 2)
    with pytest.raises(ValueError):
        topk_probs(np.full((1, 4), -math.inf), 1)


# --- planted mistakes: each must fail one of the pins above -------------------------
def _mut_renormalise(x, K):
    idx, p, lse = topk_probs(x, K)
    return idx, p / p.sum(axis=1, keepdims=True), lse


def _mut_ties_by_larger_index(x, K):
    x = np.asarray(x, np.float64)
    V = x.shape[1]
    order = (V - 1 - np.argsort(-x[:, ::-1], axis=1, kind="stable"))[:, :K]
    idx, p, lse = topk_probs(x, K)
    return order.astype(np.int32), np.exp(np.take_along_axis(x, order, 1) - lse[:, None]), lse


def _mut_lse_without_max(x, K):
    idx, p, lse = topk_probs(x, K)
    x = np.asarray(x, np.float64)
    lse2 = np.log(np.exp(x[:, :-1]).sum(axis=1))   # drops the last vocabulary entry
    return idx, np.exp(np.take_along_axis(x, idx, 1) - lse2[:, None]), lse2


@pytest.mark.parametrize("mut", [_mut_renormalise, _mut_ties_by_larger_index, _mut_lse_without_max])
def test_planted_mistakes_are_caught(mut):
    caught = False
    x = np.array([[0.0, math.log(2), math.log(3), -math.inf, math.log(2)]])
    idx, p, lse = mut(x, 5)
    caught |= idx.tolist() != [[2, 1, 4, 0, 3]] or not np.allclose(p, [[3 / 8, 2 / 8, 2 / 8, 1 / 8, 0]])
    x = np.array([[1.0, 2.0, 2.0, 0.0, -0.0, 2.0, -1.0, 0.0]])
    idx, p, _ = mut(x, 4)
    bi, bp = _brute(x[0].tolist(), 4)
    caught |= idx[0].tolist() != bi or not np.allclose(p[0], bp)
    assert caught
