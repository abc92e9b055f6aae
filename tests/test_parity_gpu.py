"""HIP path against the CPU oracle, element by element, on the same seeded inputs.

Small and ragged shapes are compared in full (several tiles, a partial last chunk,
V and d off the tile grid), and so are the 4096- and 32768-token workloads at
d=3072, V=128256, K=100 (loss, dh, dW and every row's loss, logsumexp and gathered
logits).  Every full-size workload, the 262144-token one included, is also compared on
512 sampled token rows (per-row loss, logsumexp, gathered logits and dh rows, with the
batch's own count) plus the whole dW of a 512-row sub-batch run through the same
kernels, and its mean loss is checked against the per-row losses the GPU returns.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, ZG_TOL, grad_err, max_abs_rel, rel, rel_fro, run, run_raw, to_device,
                      to_f64)

pytestmark = pytest.mark.gpu


def _check_full(inp, got, dtype=None):
    dtype = dtype or inp.cfg.dtype
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL[dtype]
    errs = dict(loss=rel(got["loss"][0], ref["loss"]),
                dh=grad_err(dtype, got["dh"], ref["dh"]),
                dW=grad_err(dtype, got["dW"], ref["dW"]),
                row_lse=max_abs_rel(got["row_lse"], ref["row_lse"]),
                zg=max_abs_rel(got["zg"], ref["zg"]),
                row_loss=max_abs_rel(got["row_loss"], ref["row_loss"]))
    print(inp.cfg.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] <= tol["loss"], errs
    assert errs["dh"] <= tol["grad"], errs
    assert errs["dW"] <= tol["grad"], errs
    assert errs["row_lse"] <= tol["loss"], errs
    assert errs["zg"] <= ZG_TOL, errs
    assert errs["row_loss"] <= 10 * tol["loss"], errs
    masked = inp.mask == 0
    if masked.any():
        assert np.all(got["dh"][masked] == 0.0)
        assert np.all(got["row_loss"][masked] == 0.0)
    return ref


def test_tiny_fp32_config_in_full(torch_cuda):
    inp = synth.make(0)
    _check_full(inp, run(inp, torch_cuda))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shapes_in_full(torch_cuda, dtype):
    """V, d and N off the tile grid, a partial last chunk, masked rows and a repeated
    teacher index (scatter-add)."""
    inp = synth.make(1, seed=77, N=700, d=264, V=3001, K=7, chunk=300, dtype=dtype)
    inp.mask[[0, 5, 299, 300, 699]] = 0
    inp.idx[3, 1] = inp.idx[3, 0]
    inp.idx[650, 6] = inp.idx[650, 2]
    _check_full(inp, run(inp, torch_cuda))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,d,N,chunk,repeat", [
    (1, 1, 8, 5, 2, False),      # one vocabulary entry: q = 1, the loss is sum p log p
    (1, 3, 8, 9, 4, True),       # one entry named three times in every row
    (2, 1, 8, 33, 7, False),     # K = 1: the loss is M times the cross-entropy
    (7, 1, 16, 300, 128, False),
    (385, 2, 64, 257, 256, False),  # one vocabulary row past a 384-row tile
])
def test_degenerate_shapes(torch_cuda, dtype, V, K, d, N, chunk, repeat):
    """Vocabularies of one and two entries, K = 1, the smallest d, a vocabulary one row
    past a tile and chunks that split the batch unevenly, in full against the oracle."""
    inp = synth.make(1, seed=1000 + V * 10 + K, N=N, d=d, V=V, K=1 if repeat else K,
                     chunk=chunk, dtype=dtype)
    if repeat:  # K entries of the only index, with probabilities that sum to M
        inp.idx = np.zeros((N, K), np.int32)
        inp.p = np.repeat(inp.p / K, K, axis=1).astype(np.float32)
        inp.cfg = dataclasses.replace(inp.cfg, K=K)
    inp.mask[N // 2] = 0
    got = run(inp, torch_cuda)
    if V > 1:
        _check_full(inp, got)
        return
    # One entry: q = 1, dz = M * 1 - (the row's p) = 0 exactly, so the gradients are zero
    # and a relative error has no scale; they must be at the rounding floor of dz (one
    # bf16 rounding of s*M, then the subtraction), i.e. below 2^-7 of s*M*|W| (bf16) or
    # 1e-6 of it (fp32); the loss, lse and gathered logits are compared as usual.
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL[dtype]
    assert rel(got["loss"][0], ref["loss"]) <= tol["loss"]
    assert max_abs_rel(got["row_lse"], ref["row_lse"]) <= tol["loss"]
    assert max_abs_rel(got["zg"], ref["zg"]) <= ZG_TOL
    count = int((inp.mask != 0).sum())
    dz_floor = (2.0 ** -7 if dtype == "bf16" else 1e-6) * K / count  # bound on |dz|
    dh_max, dW_max = float(np.abs(got["dh"]).max()), float(np.abs(got["dW"]).max())
    print(dtype, "V=1 dh", dh_max, "dW", dW_max, flush=True)
    assert dh_max <= dz_floor * np.abs(inp.W64()).max()     # dh = dz * W[0]
    assert dW_max <= dz_floor * np.abs(inp.h64()).max() * N  # dW[0] = sum_n dz[n] h[n]


def test_token_tile_groups_with_a_partial_group(torch_cuda):
    """A chunk of eleven 256-token tiles: the logits GEMMs take token tiles in groups of
    eight, so the chunk has one whole group and a partial one of three (with a partial
    last token tile), over several vocabulary tiles; in full against the oracle, for the
    one call and for the split pair (whose recompute GEMM takes the same order)."""
    inp = synth.make(1, seed=81, N=2700, d=128, V=2500, K=9, chunk=2700)
    inp.mask[[1, 2048, 2699]] = 0
    got = run(inp, torch_cuda)
    ref = _check_full(inp, got)
    split = _run_split(inp, torch_cuda)
    tol = TOL["bf16"]
    assert rel(split["loss"][0], ref["loss"]) <= tol["loss"]
    assert grad_err("bf16", split["dh"], ref["dh"]) <= tol["grad"]
    assert grad_err("bf16", split["dW"], ref["dW"]) <= tol["grad"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_logit_range(torch_cuda, dtype):
    """Logits with a standard deviation near 60: for most 192-row vocabulary groups of a
    token exp(group max - lse) underflows to zero, so the fused call's kept exponentials
    are scaled by zero there and teacher entries in those groups leave the sparse term
    alone in dz."""
    inp = synth.make(1, seed=21, N=300, d=128, V=5000, K=12, chunk=128, dtype=dtype)
    if dtype == "bf16":
        inp.W = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.W) * 30.0)
    else:
        inp.W = (inp.W * 30.0).astype(np.float32)
    _check_full(inp, run(inp, torch_cuda))


def test_dh_split_over_several_rounds(torch_cuda):
    """d = 3136 needs nine 384-row tiles of dh per 256-token tile, so the vocabulary is
    split seven ways and the dh GEMM runs 504 workgroups, two rounds of the 256 CUs (the
    last d tile partial); the float32 partials are reduced in order."""
    inp = synth.make(1, seed=61, N=2048, d=3136, V=16000, K=20, chunk=2048)
    inp.mask[[1, 1000, 2047]] = 0
    _check_full(inp, run(inp, torch_cuda))


def _uniform_teacher(N, V, K, rng):
    """K distinct uniform indices per row (a permutation when K = V) and probabilities
    from the softmax of sorted N(0, 2) scores, scaled to a mass of 0.9."""
    idx = np.argsort(rng.random((N, V)), axis=1)[:, :K].astype(np.int32)
    sc = -np.sort(-rng.normal(0.0, np.sqrt(2.0), (N, K)), axis=1)
    e = np.exp(sc - sc[:, :1])
    return idx, (0.9 * e / e.sum(axis=1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("dtype,V,K", [("bf16", 3001, 300), ("f32", 2000, 1100),
                                       ("bf16", 700, 700)])
def test_large_k(torch_cuda, dtype, V, K):
    """K above the 256 indices a scatter wave hashes (so every row takes the path that
    sums repeats first), up to K = V; some rows repeat entries, one of them many times."""
    rng = np.random.default_rng(40 + K)
    inp = synth.make(1, seed=41, N=300, d=72, V=V, K=4, chunk=128, dtype=dtype)
    inp.idx, inp.p = _uniform_teacher(300, V, K, rng)
    inp.idx[5, 1] = inp.idx[5, 0]
    inp.idx[200, K - 1] = inp.idx[200, 3]
    inp.idx[201, : K // 2] = inp.idx[201, K - 1]
    inp.mask[[7, 150]] = 0
    _check_full(inp, run(inp, torch_cuda))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_teacher_entries_than_vocabulary(torch_cuda, dtype):
    """K > V is valid (repeated indices): 120 entries per row over a 50-token vocabulary,
    drawn with replacement, so every row repeats indices; the gather reads each entry and
    the sparse term adds the probabilities of equal indices."""
    rng = np.random.default_rng(71)
    N, V, K = 200, 50, 120
    inp = synth.make(1, seed=72, N=N, d=40, V=V, K=4, chunk=64, dtype=dtype)
    inp.idx = rng.integers(0, V, size=(N, K)).astype(np.int32)
    sc = -np.sort(-rng.normal(0.0, np.sqrt(2.0), (N, K)), axis=1)
    e = np.exp(sc - sc[:, :1])
    inp.p = (0.95 * e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    inp.mask[[3, 100]] = 0
    _check_full(inp, run(inp, torch_cuda))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_student_equal_to_teacher_gives_zero(torch_cuda, dtype):
    """K = V with the teacher's probabilities equal to the student's softmax (from the
    oracle's logits of the same inputs): the loss and both gradients vanish, up to
    rounding, against the gradients of a random teacher.  In bf16 the floor is dz's own
    rounding (2^-9 of each M*softmax entry, which the exact p no longer cancels): about
    7e-4 of the random teacher's gradients; fp32 reaches about 3e-7."""
    N, V = 200, 600
    rng = np.random.default_rng(50)
    inp = synth.make(1, seed=51, N=N, d=64, V=V, K=4, chunk=64, dtype=dtype)
    Z = inp.h64() @ inp.W64().T
    q = np.exp(Z - Z.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    inp.idx = np.argsort(rng.random((N, V)), axis=1).astype(np.int32)
    inp.p = np.take_along_axis(q, inp.idx, axis=1).astype(np.float32)
    got = run(inp, torch_cuda)
    scale = run(synth.make(1, seed=51, N=N, d=64, V=V, K=8, chunk=64, dtype=dtype), torch_cuda)
    print(dtype, "loss", got["loss"][0], "max row loss", np.abs(got["row_loss"]).max(),
          "dh ratio", np.linalg.norm(got["dh"]) / np.linalg.norm(scale["dh"]),
          "dW ratio", np.linalg.norm(got["dW"]) / np.linalg.norm(scale["dW"]), flush=True)
    assert abs(got["loss"][0]) < 1e-5
    assert np.abs(got["row_loss"]).max() < 2e-5
    floor = 5e-3 if dtype == "bf16" else 1e-5
    assert np.linalg.norm(got["dh"]) < floor * np.linalg.norm(scale["dh"])
    assert np.linalg.norm(got["dW"]) < floor * np.linalg.norm(scale["dW"])


def test_tiny_chunks_and_single_token(torch_cuda):
    inp = synth.make(0, seed=5, N=37, d=8, V=300, K=3, chunk=1, dtype="bf16")
    _check_full(inp, run(inp, torch_cuda))
    one = synth.make(0, seed=6, N=1, d=16, V=5, K=5, chunk=4, dtype="f32")
    _check_full(one, run(one, torch_cuda))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_probe_is_bit_exact(torch_cuda, dtype):
    """h_n = (2^16, 2^8, 1, 0, ...), W[j] = (j >> 16, (j >> 8) & 255, j & 255, 0, ...):
    every value is exact in bf16 and every partial sum is an exact fp32 integer, so
    z[n, j] = j in any summation order and the gathered logits must equal the indices."""
    N, d, V, K = 300, 16, 70001, 24
    inp = synth.make(0, seed=9, N=N, d=d, V=V, K=K, chunk=128, dtype=dtype)
    h = np.zeros((N, d), np.float32); h[:, 0] = 2.0**16; h[:, 1] = 2.0**8; h[:, 2] = 1.0
    j = np.arange(V)
    W = np.zeros((V, d), np.float32)
    W[:, 0] = j >> 16; W[:, 1] = (j >> 8) & 255; W[:, 2] = j & 255
    if dtype == "bf16":
        inp.h, inp.W = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(W)
    else:
        inp.h, inp.W = h, W
    got = run(inp, torch_cuda)
    assert np.array_equal(got["zg"], inp.idx.astype(np.float64))


def test_chunk_invariance_and_determinism(torch_cuda):
    inp = synth.make(1, seed=11, N=520, d=128, V=5000, K=9, chunk=64)
    runs = [run(inp, torch_cuda, chunk=c) for c in (64, 128, 1000, 520)]
    again = run(inp, torch_cuda, chunk=64)
    for k in ("loss", "dh", "dW", "row_lse", "zg"):
        assert np.array_equal(runs[0][k], again[k]), f"{k} not bitwise reproducible"
    for r in runs[1:]:
        assert rel(r["loss"][0], runs[0]["loss"][0]) < 1e-5
        assert rel_fro(r["dh"], runs[0]["dh"]) < 1e-2
        assert rel_fro(r["dW"], runs[0]["dW"]) < 1e-2
        np.testing.assert_array_equal(r["zg"], runs[0]["zg"])


def test_all_masked_and_empty(torch_cuda):
    inp = synth.make(0, seed=12, N=40, d=32, V=700, K=5, chunk=16)
    inp.mask[:] = 0
    got = run(inp, torch_cuda)
    assert got["loss"][0] == 0.0 and not got["dh"].any() and not got["dW"].any()
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    assert max_abs_rel(got["row_lse"], ref["row_lse"]) < 1e-5
    assert not got["row_loss"].any()
    empty = synth.make(0, seed=13, N=0, d=32, V=700, K=5, chunk=16)
    got = run(empty, torch_cuda)
    assert got["loss"][0] == 0.0 and not got["dW"].any() and got["dh"].shape == (0, 32)


@pytest.mark.parametrize("bad", ["idx_high", "idx_negative", "p_negative", "p_nan", "p_inf"])
def test_invalid_teacher_entry_is_rejected_with_outputs_untouched(torch_cuda, bad):
    torch = torch_cuda
    import output_head_kl_amd as kd
    inp = synth.make(0, seed=14, N=64, d=32, V=500, K=4, chunk=32)
    if bad == "idx_high":
        inp.idx[17, 2] = 500
    elif bad == "idx_negative":
        inp.idx[63, 0] = -3
    elif bad == "p_negative":
        inp.p[1, 1] = -1e-3
    elif bad == "p_nan":
        inp.p[40, 3] = np.nan
    else:
        inp.p[0, 0] = np.inf
    h, W, idx, p, mask = to_device(inp, torch)
    lib = kd._lib()
    loss = torch.full((1,), 7.0, device="cuda")
    dh = torch.full((64, 32), 7.0, device="cuda")
    dW = torch.full((500, 32), 7.0, device="cuda")
    ws = torch.empty(kd.workspace_bytes(64, 32, 500, 4, 32, kd.KD_F32), dtype=torch.uint8,
                     device="cuda")
    rc = lib.kd_chunked_kl_fwd_bwd(h.data_ptr(), W.data_ptr(), kd.KD_F32, idx.data_ptr(),
                                   p.data_ptr(), mask.data_ptr(), 64, 32, 500, 4, 32,
                                   loss.data_ptr(), dh.data_ptr(), dW.data_ptr(), None, None,
                                   None, ws.data_ptr(), ws.numel(),
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 2, lib.kd_last_error()
    assert bool((loss == 7.0).all() and (dh == 7.0).all() and (dW == 7.0).all())


def test_gradient_invariants_on_gpu(torch_cuda):
    """sum_v dW[v, :] = 0; a constant column of W gives a zero column of dh;
    <dh, h> = <dW, W>."""
    inp = synth.make(1, seed=15, N=300, d=64, V=4000, K=10, chunk=128, dtype="f32")
    inp.W[:, 5] = 0.25
    got = run(inp, torch_cuda)
    scale = np.abs(got["dW"]).max()
    assert np.abs(got["dW"].sum(0)).max() < 1e-4 * scale * np.sqrt(4000)
    assert np.abs(got["dh"][:, 5]).max() < 1e-4 * np.abs(got["dh"]).max()
    a = float(np.sum(got["dh"] * inp.h64()))
    b = float(np.sum(got["dW"] * inp.W64()))
    assert abs(a - b) <= 1e-4 * max(abs(a), abs(b))


@pytest.mark.parametrize("group", [0, 1100, 1600])
def test_smaller_dw_group_workspace(torch_cuda, group):
    """A workspace sized for a smaller dW group (one, two or three 300-token chunks of
    five, so the last group is partial) gives the fused call's loss, row outputs and dh
    bit for bit, and dW within the tolerance; the backward half likewise."""
    torch = torch_cuda
    import output_head_kl_amd as kd
    inp = synth.make(1, seed=31, N=1500, d=136, V=3001, K=7, chunk=300, dtype="bf16")
    inp.mask[[3, 700, 1499]] = 0
    base = run(inp, torch)
    got = run(inp, torch, dw_group_tokens=group)
    for k in ("loss", "dh", "row_loss", "row_lse", "zg"):
        assert np.array_equal(got[k], base[k]), k
    ref = _check_full(inp, got)
    assert rel_fro(got["dW"], base["dW"]) < 1e-5
    h, W, idx, p, mask = to_device(inp, torch)
    lse = torch.from_numpy(ref["row_lse"].astype(np.float32)).cuda()
    dh_a, dW_a = kd.bwd(h, W, idx, p, lse, None, mask, chunk=300)
    dh_b, dW_b = kd.bwd(h, W, idx, p, lse, None, mask, chunk=300, dw_group_tokens=group)
    assert bool(torch.equal(dh_a, dh_b))
    assert rel_fro(to_f64(dW_b, torch), ref["dW"]) <= TOL["bf16"]["grad"]
    assert rel_fro(to_f64(dW_b, torch), to_f64(dW_a, torch)) < 1e-5


def test_workspace_below_one_chunk_group_is_rejected(torch_cuda):
    torch = torch_cuda
    import output_head_kl_amd as kd
    inp = synth.make(1, seed=32, N=600, d=64, V=1000, K=4, chunk=200, dtype="bf16")
    h, W, idx, p, mask = to_device(inp, torch)
    need = kd.workspace_bytes(600, 64, 1000, 4, 200, dw_group_tokens=0)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kd.KDError, match="KD_E_WORKSPACE"):
        kd.fwd_bwd(h, W, idx, p, mask, chunk=200, workspace=ws)


# ------------------------------------------------------------------ full-size workloads
def _run_split(inp, torch, chunk=None, rows=None):
    """The forward and backward halves (kd_chunked_kl_fwd, then kd_chunked_kl_bwd with
    g = 1 and the saved logsumexp), as float64 numpy: loss, row outputs and, for the
    selected token rows (all when None), dh; dW whole."""
    import output_head_kl_amd as kd
    h, W, idx, p, mask = to_device(inp, torch)
    chunk = chunk or inp.cfg.chunk
    loss, row_lse, row_loss, zg = kd.fwd(h, W, idx, p, mask, chunk=chunk, rows=True)
    dh, dW = kd.bwd(h, W, idx, p, row_lse, None, mask, chunk=chunk)
    torch.cuda.synchronize()
    if rows is not None:
        dh = dh.index_select(0, torch.from_numpy(rows).cuda())
    out = dict(loss=to_f64(loss, torch), row_lse=to_f64(row_lse, torch),
               row_loss=to_f64(row_loss, torch), zg=to_f64(zg, torch), dh=to_f64(dh, torch),
               dW=to_f64(dW, torch))
    del h, W, idx, p, mask, loss, row_lse, row_loss, zg, dh, dW
    return out


_CACHE = {}


def _full(cid):
    if cid not in _CACHE:
        _CACHE.clear()
        _CACHE[cid] = synth.make(cid)
    return _CACHE[cid]


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_full_size_workload_on_sampled_rows(torch_cuda, cid):
    torch = torch_cuda
    inp = _full(cid)
    cfg = inp.cfg
    print(f"config {cid} {cfg.name}: N={cfg.N} d={cfg.d} V={cfg.V} K={cfg.K} chunk={cfg.chunk}",
          flush=True)
    raw = run_raw(inp, torch, rows=True)
    rows = synth.subset_rows(cfg, inp.seed, 512)
    sel = torch.from_numpy(rows).cuda()
    got = {k: to_f64(raw[k], torch) for k in ("loss", "row_loss", "row_lse", "zg")}
    got["dh"] = to_f64(raw["dh"].index_select(0, sel), torch)
    dh_masked_zero = bool((raw["dh"][torch.from_numpy(inp.mask == 0).cuda()] == 0).all())
    del raw
    count = int((inp.mask != 0).sum())
    # the mean loss is the masked mean of the per-row losses the GPU returns
    assert rel(got["loss"][0], got["row_loss"].sum() / count) < 1e-5
    ref = oracle.rows_forward_backward(inp.h64(rows), inp.W64(), inp.idx[rows], inp.p[rows],
                                       inp.mask[rows], count)
    tol = TOL[cfg.dtype]
    errs = dict(row_loss=rel_fro(got["row_loss"][rows], ref["row_loss"]),
                row_lse=max_abs_rel(got["row_lse"][rows], ref["row_lse"]),
                zg=rel_fro(got["zg"][rows], ref["zg"]),
                dh=rel_fro(got["dh"], ref["dh"]))
    print(f"config {cid} sampled rows:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["row_loss"] <= tol["loss"], errs
    assert errs["row_lse"] <= tol["loss"], errs
    assert errs["zg"] <= ZG_TOL, errs
    assert errs["dh"] <= tol["grad"], errs
    assert dh_masked_zero
    del got
    # the same rows from the forward and backward halves (logits recomputed)
    sp = _run_split(inp, torch, rows=rows)
    errs = dict(loss=rel(sp["loss"][0], sp["row_loss"].sum() / count),
                row_loss=rel_fro(sp["row_loss"][rows], ref["row_loss"]),
                row_lse=max_abs_rel(sp["row_lse"][rows], ref["row_lse"]),
                zg=rel_fro(sp["zg"][rows], ref["zg"]), dh=rel_fro(sp["dh"], ref["dh"]))
    print(f"config {cid} sampled rows, fwd + bwd halves:",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] < 1e-5 and errs["row_loss"] <= tol["loss"], errs
    assert errs["row_lse"] <= tol["loss"] and errs["zg"] <= ZG_TOL, errs
    assert errs["dh"] <= tol["grad"], errs
    del sp
    # dW (and the loss) of a 512-row sub-batch through the same kernels, over two chunks,
    # from the one-call form and from the two halves
    sub = synth.take_rows(inp, rows)
    ref = oracle.forward_backward(sub.h64(), sub.W64(), sub.idx, sub.p, sub.mask)
    for form, gs in (("one call", run(sub, torch, chunk=256, rows=True)),
                     ("fwd + bwd halves", _run_split(sub, torch, chunk=256))):
        errs = dict(loss=rel(gs["loss"][0], ref["loss"]), dW=rel_fro(gs["dW"], ref["dW"]),
                    dh=rel_fro(gs["dh"], ref["dh"]))
        print(f"config {cid} sub-batch, {form}:", {k: f"{v:.2e}" for k, v in errs.items()},
              flush=True)
        assert errs["loss"] <= tol["loss"], errs
        assert errs["dW"] <= tol["grad"], errs
        assert errs["dh"] <= tol["grad"], errs


# ------------------------------------------------- the 4K- and 32K-token workloads in full
# Rows are independent, so the oracle's batch is taken in equal row parts: a part's own
# call weighs its rows by 1/count_part, and multiplying its dh rows, dW and summed loss by
# count_part/count gives that part's exact share of the whole batch's mean.  Each part is a
# test of its own (about half a minute of host time each) and checks its rows; the last
# part adds up every part's dW and loss and checks the batch's totals.
_PARTS = {1: 1, 2: 4}
_STATE = {}


def _state(torch, cid):
    st = _STATE.get(cid)
    if st is None:
        _STATE.clear()
        inp = synth.make(cid)
        got = run(inp, torch, rows=True)
        split = _run_split(inp, torch)
        st = dict(inp=inp, got=got, split=split, h64=inp.h64(), W64=inp.W64(),
                  count=int((inp.mask != 0).sum()), parts={})
        _STATE[cid] = st
    return st


def _part(st, cid, q):
    if q not in st["parts"]:
        inp, n = st["inp"], st["inp"].cfg.N // _PARTS[cid]
        r0, r1 = q * n, (q + 1) * n if q + 1 < _PARTS[cid] else inp.cfg.N
        ref = oracle.forward_backward(st["h64"][r0:r1], st["W64"], inp.idx[r0:r1],
                                      inp.p[r0:r1], inp.mask[r0:r1], block_rows=128)
        w = ref["count"] / st["count"]
        st["parts"][q] = dict(r0=r0, r1=r1, dh=ref["dh"] * w, dW=ref["dW"] * w,
                              loss_sum=ref["loss"] * ref["count"], row_loss=ref["row_loss"],
                              row_lse=ref["row_lse"], zg=ref["zg"])
    return st["parts"][q]


@pytest.mark.parametrize("cid,part", [(1, 0)] + [(2, q) for q in range(_PARTS[2])])
def test_workload_in_full(torch_cuda, cid, part):
    """Both forms against the oracle: the one-call kd_chunked_kl_fwd_bwd and the forward
    and backward halves (kd_chunked_kl_fwd, then kd_chunked_kl_bwd with g = 1)."""
    st = _state(torch_cuda, cid)
    cfg, tol = st["inp"].cfg, TOL[st["inp"].cfg.dtype]
    ref = _part(st, cid, part)
    r0, r1 = ref["r0"], ref["r1"]
    masked = st["inp"].mask[r0:r1] == 0
    for form, got in (("one call", st["got"]), ("fwd + bwd halves", st["split"])):
        errs = dict(row_loss=rel_fro(got["row_loss"][r0:r1], ref["row_loss"]),
                    row_lse=max_abs_rel(got["row_lse"][r0:r1], ref["row_lse"]),
                    zg=rel_fro(got["zg"][r0:r1], ref["zg"]),
                    dh=rel_fro(got["dh"][r0:r1], ref["dh"]))
        print(f"config {cid} {cfg.name} rows {r0}..{r1}, {form}:",
              {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        assert errs["row_loss"] <= tol["loss"], errs
        assert errs["row_lse"] <= tol["loss"], errs
        assert errs["zg"] <= ZG_TOL, errs
        assert errs["dh"] <= tol["grad"], errs
        assert np.all(got["dh"][r0:r1][masked] == 0.0)
    if part + 1 < _PARTS[cid]:
        return
    parts = [_part(st, cid, q) for q in range(_PARTS[cid])]
    dW = parts[0]["dW"]
    for x in parts[1:]:
        dW += x["dW"]
    loss = sum(x["loss_sum"] for x in parts) / st["count"]
    dh = np.concatenate([x["dh"] for x in parts])
    results = {}
    for form, got in (("one call", st["got"]), ("fwd + bwd halves", st["split"])):
        results[form] = dict(loss=rel(got["loss"][0], loss), dh=rel_fro(got["dh"], dh),
                             dW=rel_fro(got["dW"], dW))
        print(f"config {cid} {cfg.name} whole batch, {form}:",
              {k: f"{v:.2e}" for k, v in results[form].items()}, flush=True)
    _STATE.clear()
    for errs in results.values():
        assert errs["loss"] <= tol["loss"], errs
        assert errs["dh"] <= tol["grad"], errs
        assert errs["dW"] <= tol["grad"], errs
