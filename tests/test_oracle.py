"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself: the
hand-derived worked examples, central finite differences of its own loss,
torch's kl_div / cross_entropy / autograd in float64, closed forms (zero
projection, student equal to teacher) and invariants of the definition.  A
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_worked.json")


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"log": math.log}))


def _arr(a):
    return np.array([[_ev(v) for v in row] for row in a]) if isinstance(a[0], list) \
        else np.array([_ev(v) for v in a])


def _rand_case(rng, N=6, d=5, V=13, K=4, distinct=True, pzero=False):
    h = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) * 0.7
    if distinct:
        idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    else:
        idx = rng.integers(0, V, size=(N, K))
    s = np.sort(rng.standard_normal((N, K)) * 1.4, axis=1)[:, ::-1]
    p = np.exp(s) / np.exp(s).sum(1, keepdims=True) * rng.uniform(0.8, 0.99, (N, 1))
    if pzero:
        p[0, -1] = 0.0
    return h, W, idx, p


def _torch_loss(h, W, idx, p, mask):
    """The loss written with torch ops (log_softmax + gather), float64."""
    z = h @ W.T
    logq = torch.log_softmax(z, dim=1)
    plogp = torch.where(p > 0, p * torch.log(torch.where(p > 0, p, torch.ones_like(p))),
                        torch.zeros_like(p))
    ell = (plogp - p * torch.gather(logq, 1, idx)).sum(1)
    m = mask.to(torch.float64)
    return (ell * m).sum() / m.sum()


# ---------------------------------------------------------------- worked examples
def test_golden_worked_examples():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        h = np.array(c["h"], dtype=np.float64)
        W = _arr(c["W"])
        out = oracle.forward_backward(h, W, np.array(c["idx"]), np.array(c["p"]),
                                      np.array(c["mask"]))
        assert out["loss"] == pytest.approx(_ev(c["loss"]), rel=1e-13, abs=1e-15), c["name"]
        np.testing.assert_allclose(out["row_lse"], _arr(c["row_lse"]), rtol=1e-13)
        np.testing.assert_allclose(out["zg"], _arr(c["zg"]), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(out["dh"], _arr(c["dh"]), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(out["dW"], _arr(c["dW"]), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("distinct,masked", [(True, False), (False, True)])
def test_gradient_matches_central_differences(distinct, masked):
    """The closed-form gradient (pages: M*softmax minus the sparse correction) equals
    central differences of the oracle's own loss, including repeated indices,
    a zero probability and a masked row."""
    rng = np.random.default_rng(7)
    h, W, idx, p = _rand_case(rng, N=6, d=5, V=13, K=4, distinct=distinct, pzero=True)
    mask = np.ones(6, dtype=np.uint8)
    if masked:
        mask[2] = 0
    out = oracle.forward_backward(h, W, idx, p, mask)
    eps = 1e-6

    def fd(x, setter):
        g = np.zeros_like(x)
        for i in np.ndindex(*x.shape):
            xp = x.copy(); xp[i] += eps
            xm = x.copy(); xm[i] -= eps
            g[i] = (setter(xp) - setter(xm)) / (2 * eps)
        return g

    gh = fd(h, lambda hh: oracle.loss_only(hh, W, idx, p, mask))
    gW = fd(W, lambda WW: oracle.loss_only(h, WW, idx, p, mask))
    scale_h = np.abs(out["dh"]).max()
    scale_W = np.abs(out["dW"]).max()
    assert np.abs(gh - out["dh"]).max() <= 1e-7 * max(scale_h, 1e-3)
    assert np.abs(gW - out["dW"]).max() <= 1e-7 * max(scale_W, 1e-3)
    if masked:
        assert np.all(out["dh"][2] == 0.0)


# ---------------------------------------------------------------- library routines
def test_loss_matches_torch_kl_div_on_densified_teacher():
    """With the teacher densified to P[n, v] (zero off the support), each token's loss is
    torch's pointwise KL, P (log P - log_softmax z), summed over the vocabulary."""
    rng = np.random.default_rng(3)
    N, d, V, K = 7, 6, 31, 5
    h, W, idx, p = _rand_case(rng, N, d, V, K, distinct=True)
    out = oracle.forward_backward(h, W, idx, p)
    P = np.zeros((N, V))
    np.put_along_axis(P, idx, p, axis=1)
    z = torch.from_numpy(h) @ torch.from_numpy(W).T
    kl = torch.nn.functional.kl_div(torch.log_softmax(z, 1), torch.from_numpy(P),
                                    reduction="none").sum(1).numpy()
    np.testing.assert_allclose(out["row_loss"], kl, rtol=1e-12, atol=1e-14)
    assert out["loss"] == pytest.approx(kl.mean(), rel=1e-12)
    np.testing.assert_allclose(out["row_lse"], torch.logsumexp(z, 1).numpy(), rtol=1e-14)


def test_single_target_reduces_to_cross_entropy():
    """K = 1 with p = 1 is the textbook cross entropy; its gradient is softmax - onehot."""
    rng = np.random.default_rng(4)
    N, d, V = 9, 4, 17
    h = rng.standard_normal((N, d)); W = rng.standard_normal((V, d))
    t = rng.integers(0, V, size=N)
    out = oracle.forward_backward(h, W, t[:, None], np.ones((N, 1)))
    ht = torch.tensor(h, requires_grad=True); Wt = torch.tensor(W, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(ht @ Wt.T, torch.from_numpy(t))
    ce.backward()
    assert out["loss"] == pytest.approx(ce.item(), rel=1e-13)
    np.testing.assert_allclose(out["dh"], ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_gradient_matches_torch_autograd():
    rng = np.random.default_rng(5)
    N, d, V, K = 11, 8, 40, 6
    h, W, idx, p = _rand_case(rng, N, d, V, K, distinct=False, pzero=True)
    mask = (rng.random(N) > 0.3).astype(np.uint8); mask[0] = 1
    out = oracle.forward_backward(h, W, idx, p, mask)
    ht = torch.tensor(h, requires_grad=True); Wt = torch.tensor(W, requires_grad=True)
    L = _torch_loss(ht, Wt, torch.from_numpy(idx), torch.from_numpy(p), torch.from_numpy(mask))
    L.backward()
    assert out["loss"] == pytest.approx(L.item(), rel=1e-13)
    np.testing.assert_allclose(out["dh"], ht.grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-15)


# ---------------------------------------------------------------- closed forms
def test_zero_projection_gives_uniform_student():
    """W = 0 makes every logit 0: lse = log V, l = sum p log p + M log V,
    dZ = s (M/V - scatter p), dh = 0, dW = dZ^T h."""
    rng = np.random.default_rng(6)
    N, d, V, K = 5, 3, 50, 7
    h, _, idx, p = _rand_case(rng, N, d, V, K)
    W = np.zeros((V, d))
    out = oracle.forward_backward(h, W, idx, p)
    assert np.all(out["row_lse"] == np.log(V))
    H = (p * np.log(p)).sum(1)
    M = p.sum(1)
    np.testing.assert_allclose(out["row_loss"], H + M * np.log(V), rtol=1e-13)
    assert np.all(out["dh"] == 0.0)
    P = np.zeros((N, V)); np.put_along_axis(P, idx, p, axis=1)
    dZ = (M[:, None] / V - P) / N
    np.testing.assert_allclose(out["dW"], dZ.T @ h, rtol=1e-12, atol=1e-16)


def test_student_equal_to_teacher_gives_zero():
    """K = V and p = softmax(z): the KL is zero and so are both gradients."""
    rng = np.random.default_rng(8)
    N, d, V = 4, 3, 9
    h = rng.standard_normal((N, d)); W = rng.standard_normal((V, d))
    z = h @ W.T
    q = np.exp(z - z.max(1, keepdims=True)); q /= q.sum(1, keepdims=True)
    idx = np.tile(np.arange(V), (N, 1))
    out = oracle.forward_backward(h, W, idx, q)
    assert abs(out["loss"]) < 1e-14
    assert np.abs(out["dh"]).max() < 1e-15
    assert np.abs(out["dW"]).max() < 1e-15


# ---------------------------------------------------------------- invariants
def test_logit_gradient_rows_sum_to_zero():
    """sum_v dZ[n, v] = s_n (M_n - sum_k p_nk) = 0, hence sum_v dW[v, :] = 0 and a
    constant column of W gives a zero column of dh."""
    rng = np.random.default_rng(9)
    N, d, V, K = 8, 6, 33, 5
    h, W, idx, p = _rand_case(rng, N, d, V, K, distinct=False)
    W[:, 2] = 0.37
    out = oracle.forward_backward(h, W, idx, p)
    assert np.abs(out["dW"].sum(0)).max() < 1e-15 * V
    assert np.abs(out["dh"][:, 2]).max() < 1e-15 * V


def test_trace_identity():
    """<dh, h> = <dW, W> = sum dZ * Z."""
    rng = np.random.default_rng(10)
    h, W, idx, p = _rand_case(rng, N=9, d=7, V=29, K=6)
    out = oracle.forward_backward(h, W, idx, p)
    a = np.sum(out["dh"] * h)
    b = np.sum(out["dW"] * W)
    assert a == pytest.approx(b, rel=1e-12)


def test_shift_invariance():
    """An extra hidden unit with W[:, j] = 1 and h[n, j] = c_n shifts row n's logits by
    c_n, which leaves softmax and the loss unchanged."""
    rng = np.random.default_rng(11)
    h, W, idx, p = _rand_case(rng, N=6, d=4, V=21, K=5)
    c = rng.standard_normal(6) * 3
    h2 = np.concatenate([h, c[:, None]], 1)
    W2 = np.concatenate([W, np.ones((21, 1))], 1)
    a = oracle.forward_backward(h, W, idx, p)
    b = oracle.forward_backward(h2, W2, idx, p)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(b["row_lse"] - c, a["row_lse"], rtol=1e-13)
    np.testing.assert_allclose(b["dh"][:, :4], a["dh"], rtol=1e-11, atol=1e-16)
    assert np.abs(b["dh"][:, 4]).max() < 1e-15


def test_mask_equals_compacted_batch():
    rng = np.random.default_rng(12)
    N = 10
    h, W, idx, p = _rand_case(rng, N=N, d=5, V=19, K=4)
    mask = np.array([1, 0, 1, 1, 0, 0, 1, 1, 1, 0], dtype=np.uint8)
    a = oracle.forward_backward(h, W, idx, p, mask)
    keep = mask != 0
    b = oracle.forward_backward(h[keep], W, idx[keep], p[keep])
    assert a["count"] == keep.sum()
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-13)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(a["dh"][keep], b["dh"], rtol=1e-12, atol=1e-16)
    assert np.all(a["dh"][~keep] == 0.0)
    assert np.all(a["row_loss"][~keep] == 0.0)


def test_permutations():
    rng = np.random.default_rng(13)
    N, d, V, K = 7, 4, 23, 5
    h, W, idx, p = _rand_case(rng, N, d, V, K)
    a = oracle.forward_backward(h, W, idx, p)
    perm = rng.permutation(N)
    b = oracle.forward_backward(h[perm], W, idx[perm], p[perm])
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(b["dh"], a["dh"][perm], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(b["dW"], a["dW"], rtol=1e-12, atol=1e-16)
    vp = rng.permutation(V)           # new row j holds old row vp[j]
    inv = np.argsort(vp)
    c = oracle.forward_backward(h, W[vp], inv[idx], p)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["dW"], a["dW"][vp], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(c["dh"], a["dh"], rtol=1e-12, atol=1e-16)


def test_row_blocking_changes_nothing():
    rng = np.random.default_rng(14)
    h, W, idx, p = _rand_case(rng, N=13, d=4, V=17, K=3)
    a = oracle.forward_backward(h, W, idx, p, block_rows=1)
    b = oracle.forward_backward(h, W, idx, p, block_rows=64)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-13, atol=1e-17)
    r = oracle.rows_forward_backward(h[[2, 5, 11]], W, idx[[2, 5, 11]], p[[2, 5, 11]],
                                     np.ones(3), count=13)
    np.testing.assert_allclose(r["dh"], b["dh"][[2, 5, 11]], rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(r["row_loss"], b["row_loss"][[2, 5, 11]], rtol=1e-14)


def test_all_masked_gives_zeros():
    rng = np.random.default_rng(15)
    h, W, idx, p = _rand_case(rng, N=4, d=3, V=11, K=2)
    out = oracle.forward_backward(h, W, idx, p, np.zeros(4))
    assert out["loss"] == 0.0 and out["count"] == 0
    assert not out["dh"].any() and not out["dW"].any()


@pytest.mark.parametrize("bad", ["neg_idx", "big_idx", "neg_p", "nan_p"])
def test_rejects_invalid_teacher_entries(bad):
    rng = np.random.default_rng(16)
    h, W, idx, p = _rand_case(rng, N=3, d=2, V=7, K=2)
    if bad == "neg_idx":
        idx[1, 0] = -1
    elif bad == "big_idx":
        idx[2, 1] = 7
    elif bad == "neg_p":
        p[0, 0] = -0.1
    else:
        p[1, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.forward_backward(h, W, idx, p)
