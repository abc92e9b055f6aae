"""Pins of the vocabulary-shard oracle (``oracle.shard``) against facts fixed outside it:
a hand-derived two-shard example, and the dense oracle (itself pinned by
test_oracle.py) reassembled from shards that tile the vocabulary: the combined
statistics give its logsumexp and loss, the dh partials sum to its dh and the shards'
dW rows stack to its dW.  Planted mistakes in the shard oracle must fail a pin."""
import inspect
import json
import math
import os
import types

import numpy as np
import pytest

import oracle
import oracle.shard as shard

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "shard_worked.json")


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"log": math.log}))


def _arr(a):
    return np.array([[_ev(v) for v in row] for row in a]) if isinstance(a[0], list) \
        else np.array([_ev(v) for v in a])


def _golden_ok(mod):
    c = json.load(open(GOLDEN))
    h, W = np.array(c["h"], float), _arr(c["W"])
    idx, p, mask, g = np.array(c["idx"]), np.array(c["p"]), np.array(c["mask"]), c["g"]
    stats = []
    ok = True
    for sh in c["shards"]:
        a, n = sh["v0"], sh["Vs"]
        m, s, pz = mod.shard_stats(h, W[a:a + n], a, idx, p)
        ok &= np.allclose(m, _arr(sh["m"]), rtol=1e-13, atol=1e-15)
        ok &= np.allclose(s, _arr(sh["s"]), rtol=1e-13, atol=1e-15)
        ok &= np.allclose(pz, _arr(sh["pz"]), rtol=1e-13, atol=1e-15)
        stats.append((m, s, pz))
    comb = mod.combine(*(np.stack([st[i] for st in stats]) for i in range(3)), p, mask)
    ok &= np.allclose(comb["row_lse"], _arr(c["row_lse"]), rtol=1e-13)
    ok &= np.allclose(comb["row_loss"], _arr(c["row_loss"]), rtol=1e-12, atol=1e-15)
    ok &= math.isclose(comb["loss"], _ev(c["loss"]), rel_tol=1e-12)
    for sh in c["shards"]:
        a, n = sh["v0"], sh["Vs"]
        dh, dW = mod.shard_backward(h, W[a:a + n], a, idx, p, comb["row_lse"], mask, g=g)
        ok &= np.allclose(dh, _arr(sh["dh_partial"]), rtol=1e-12, atol=1e-15)
        ok &= np.allclose(dW, _arr(sh["dW"]), rtol=1e-12, atol=1e-15)
    return bool(ok)


def _case(seed, N=9, d=6, V=23, K=5):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) * 0.8
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    idx[2, 1] = idx[2, 0]                       # a repeated index
    s = np.sort(rng.standard_normal((N, K)), axis=1)[:, ::-1]
    p = np.exp(s) / np.exp(s).sum(1, keepdims=True) * 0.9
    p[4, -1] = 0.0                              # p = 0 contributes nothing
    mask = np.ones(N, dtype=np.uint8)
    mask[[1, 7]] = 0
    return h, W, idx, p, mask


def _reassembled_ok(mod, bounds=((0, 5), (5, 6), (6, 17), (17, 23)), g=1.7):
    """Shards that tile the vocabulary reproduce the dense oracle."""
    h, W, idx, p, mask = _case(31)
    ref = oracle.forward_backward(h, W, idx, p, mask)
    st = [mod.shard_stats(h, W[a:b], a, idx, p) for a, b in bounds]
    comb = mod.combine(*(np.stack([x[i] for x in st]) for i in range(3)), p, mask)
    ok = math.isclose(comb["loss"], ref["loss"], rel_tol=1e-12)
    ok &= np.allclose(comb["row_lse"], ref["row_lse"], rtol=1e-13)
    ok &= np.allclose(comb["row_loss"], ref["row_loss"], rtol=1e-12, atol=1e-14)
    dh = np.zeros_like(ref["dh"])
    dWs = []
    for a, b in bounds:
        dhp, dWp = mod.shard_backward(h, W[a:b], a, idx, p, comb["row_lse"], mask, g=g)
        dh += dhp
        dWs.append(dWp)
    ok &= np.allclose(dh, g * ref["dh"], rtol=1e-11, atol=1e-14)
    ok &= np.allclose(np.concatenate(dWs), g * ref["dW"], rtol=1e-11, atol=1e-14)
    return bool(ok)


def test_golden_two_shard_example():
    assert _golden_ok(shard)


@pytest.mark.parametrize("bounds", [((0, 23),), ((0, 11), (11, 23)),
                                    ((0, 5), (5, 6), (6, 17), (17, 23)),
                                    tuple((v, v + 1) for v in range(23))])
def test_shards_reassemble_the_dense_oracle(bounds):
    assert _reassembled_ok(shard, bounds)


def test_one_shard_statistics_are_the_dense_lse_and_gather():
    h, W, idx, p, mask = _case(32)
    ref = oracle.forward_backward(h, W, idx, p, mask)
    m, s, pz = shard.shard_stats(h, W, 0, idx, p)
    np.testing.assert_allclose(m + np.log(s), ref["row_lse"], rtol=1e-13)
    np.testing.assert_allclose(pz, (p * ref["zg"]).sum(1), rtol=1e-12, atol=1e-14)


def test_selected_rows_match_all_rows():
    h, W, idx, p, mask = _case(33)
    lse = oracle.forward_backward(h, W, idx, p, mask)["row_lse"]
    full, dW = shard.shard_backward(h, W[4:15], 4, idx, p, lse, mask, block_rows=4)
    rows = np.array([8, 0, 3])
    part, dW2 = shard.shard_backward(h, W[4:15], 4, idx, p, lse, mask, rows=rows, block_rows=4)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dW2, dW, rtol=1e-14, atol=1e-16)


MUTANTS = {
    "pz_counts_entries_outside_the_shard": (
        "pz[r0:r1] = np.where(inside, p[r0:r1] * z_at, 0.0).sum(axis=1)",
        "pz[r0:r1] = (p[r0:r1] * z_at).sum(axis=1)"),
    "combine_drops_the_shard_max": (
        "lse = top + np.log((ss * np.exp(ms - top[None, :])).sum(axis=0))",
        "lse = top + np.log(ss.sum(axis=0))"),
    "backward_uses_the_shard_lse": (
        "* np.exp(Z - lse[r0:r1, None])",
        "* np.exp(Z - (Z.max(1) + np.log(np.exp(Z - Z.max(1)[:, None]).sum(1)))[:, None])"),
    "scatter_index_not_localised": (
        "(rr[inside], ib[inside] - v0)", "(rr[inside], np.minimum(ib[inside], Vs - 1))"),
    "upstream_gradient_ignored": ("scale = g * mask / count", "scale = mask / count"),
    "combine_adds_pz": ("- pzs.sum(axis=0) +", "+ pzs.sum(axis=0) +"),
}


def _mutant(name):
    src = inspect.getsource(shard)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("shard_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"):
        verdicts = {"golden": _golden_ok(mod), "reassembled": _reassembled_ok(mod)}
    assert not all(verdicts.values()), f"mutant {name} survived: {verdicts}"
