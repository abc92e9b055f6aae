"""Planted mistakes in the oracle (CPU only) must be caught by its pins.

Each mutant is the oracle's source with one plausible slip edited in; the test
asserts that at least one independent pin (hand-derived worked examples, torch
kl_div, torch autograd) rejects it while the real oracle passes all of them.
"""
import inspect
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_worked.json")

MUTANTS = {
    "drop_mass_in_dense_term": ("dZ = (scale_b * M)[:, None] * np.exp(logq)",
                                "dZ = scale_b[:, None] * np.exp(logq)"),
    "flip_sparse_correction_sign": ("-(scale_b[:, None] * p_b)", "(scale_b[:, None] * p_b)"),
    "drop_teacher_entropy": ("ell = (plogp - p_b * logq_at)", "ell = (- p_b * logq_at)"),
    "drop_max_in_lse": ("lse = m + np.log", "lse = np.log"),
    "gather_off_by_one": ("logq_at = np.take_along_axis(logq, idx_b, axis=1)",
                          "logq_at = np.take_along_axis(logq, (idx_b + 1) % logq.shape[1], axis=1)"),
    "normalise_over_support_only": (
        "np.log(np.exp(Z - m[:, None]).sum(axis=1))",
        "np.log(np.exp(np.take_along_axis(Z, idx_b, axis=1) - m[:, None]).sum(axis=1))"),
    "dh_from_transposed_weight_rows": ("out[\"dh\"][r0:r1] = dZ @ W",
                                       "out[\"dh\"][r0:r1] = dZ @ W[::-1]"),
}


def _mutant(name):
    src = inspect.getsource(oracle)
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def _ev(x):
    return float(eval(x, {"__builtins__": {}}, {"log": math.log})) if isinstance(x, str) else float(x)


def _golden_ok(mod):
    for c in json.load(open(GOLDEN))["cases"]:
        W = np.array([[_ev(v) for v in r] for r in c["W"]])
        out = mod.forward_backward(np.array(c["h"], float), W, np.array(c["idx"]),
                                   np.array(c["p"]), np.array(c["mask"]))
        dh = np.array([[_ev(v) for v in r] for r in c["dh"]])
        dW = np.array([[_ev(v) for v in r] for r in c["dW"]])
        if not (math.isclose(out["loss"], _ev(c["loss"]), rel_tol=1e-12, abs_tol=1e-14)
                and np.allclose(out["dh"], dh, rtol=1e-11, atol=1e-14)
                and np.allclose(out["dW"], dW, rtol=1e-11, atol=1e-14)):
            return False
    return True


def _case(seed=21, N=7, d=5, V=19, K=4):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, d)); W = rng.standard_normal((V, d)) * 0.8
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    s = np.sort(rng.standard_normal((N, K)), axis=1)[:, ::-1]
    p = np.exp(s) / np.exp(s).sum(1, keepdims=True) * 0.9
    return h, W, idx, p


def _kl_div_ok(mod):
    h, W, idx, p = _case()
    out = mod.forward_backward(h, W, idx, p)
    P = np.zeros((h.shape[0], W.shape[0])); np.put_along_axis(P, idx, p, axis=1)
    z = torch.from_numpy(h @ W.T)
    kl = torch.nn.functional.kl_div(torch.log_softmax(z, 1), torch.from_numpy(P),
                                    reduction="none").sum(1).numpy()
    return bool(np.allclose(out["row_loss"], kl, rtol=1e-11, atol=1e-13))


def _autograd_ok(mod):
    h, W, idx, p = _case(seed=22)
    out = mod.forward_backward(h, W, idx, p)
    ht = torch.tensor(h, requires_grad=True); Wt = torch.tensor(W, requires_grad=True)
    logq = torch.log_softmax(ht @ Wt.T, 1)
    pt = torch.from_numpy(p)
    L = ((pt * torch.log(pt) - pt * torch.gather(logq, 1, torch.from_numpy(idx))).sum(1)).mean()
    L.backward()
    return bool(np.allclose(out["dh"], ht.grad.numpy(), rtol=1e-10, atol=1e-14)
                and np.allclose(out["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-14))


def test_real_oracle_passes_every_pin():
    assert _golden_ok(oracle) and _kl_div_ok(oracle) and _autograd_ok(oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"):
        verdicts = {"golden": _golden_ok(mod), "kl_div": _kl_div_ok(mod),
                    "autograd": _autograd_ok(mod)}
    assert not all(verdicts.values()), f"mutant {name} survived: {verdicts}"
