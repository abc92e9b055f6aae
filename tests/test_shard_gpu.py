"""Vocabulary shards through the C ABI: G shards of W run forward, the statistics are
combined, each shard runs backward, and the reassembled loss, logsumexp, dh (sum of
the float32 partials) and dW (the shards' rows) match the oracle of the whole head."""
import numpy as np
import pytest

import oracle
import oracle.shard as oshard
import synth
from gpu_util import TOL, grad_err, max_abs_rel, rel, rel_fro, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run_shards(inp, bounds, torch, chunk, g=None):
    import output_head_kl_amd as kd
    h, W, idx, p, mask = to_device(inp, torch)
    V = inp.cfg.V
    stats = [kd.vocab_shard_fwd(h, W[a:b].contiguous(), idx, p, a, V, chunk=chunk)
             for a, b in bounds]
    m, s, pz = (torch.stack([st[i] for st in stats]) for i in range(3))
    loss, row_lse, row_loss = kd.vocab_shard_combine(m, s, pz, p, mask)
    gt = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    dh = torch.zeros((inp.cfg.N, inp.cfg.d), dtype=torch.float32, device="cuda")
    dWs = []
    for a, b in bounds:
        dhp, dWp = kd.vocab_shard_bwd(h, W[a:b].contiguous(), idx, p, row_lse, a, V, gt, mask,
                                      chunk=chunk)
        dh += dhp            # the all-reduce of the partials (test side)
        dWs.append(dWp)
    torch.cuda.synchronize()
    return dict(loss=to_f64(loss, torch), row_lse=to_f64(row_lse, torch),
                row_loss=to_f64(row_loss, torch), dh=to_f64(dh, torch),
                dW=to_f64(torch.cat(dWs), torch))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_four_uneven_shards_match_the_whole_head(torch_cuda, dtype):
    inp = synth.make(1, seed=61, N=700, d=264, V=3001, K=7, chunk=300, dtype=dtype)
    inp.mask[[0, 5, 299, 300, 699]] = 0
    inp.idx[3, 1] = inp.idx[3, 0]          # a repeated index (scatter-add within a shard)
    bounds = [(0, 700), (700, 1500), (1500, 2600), (2600, 3001)]
    got = _run_shards(inp, bounds, torch_cuda, chunk=300)
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL[dtype]
    errs = dict(loss=rel(got["loss"][0], ref["loss"]),
                lse=max_abs_rel(got["row_lse"], ref["row_lse"]),
                row_loss=max_abs_rel(got["row_loss"], ref["row_loss"]),
                dh=grad_err(dtype, got["dh"], ref["dh"]),
                dW=grad_err(dtype, got["dW"], ref["dW"]))
    print(dtype, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] <= tol["loss"] and errs["lse"] <= tol["loss"], errs
    assert errs["row_loss"] <= 10 * tol["loss"], errs
    assert errs["dh"] <= tol["grad"] and errs["dW"] <= tol["grad"], errs
    assert np.all(got["dh"][inp.mask == 0] == 0.0)


def test_one_shard_is_the_fused_call(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(0, seed=12, N=400, chunk=128)
    got = _run_shards(inp, [(0, inp.cfg.V)], torch, chunk=128)
    h, W, idx, p, mask = to_device(inp, torch)
    loss, dh, dW = kd.fwd_bwd(h, W, idx, p, mask, chunk=128)
    torch.cuda.synchronize()
    assert rel(got["loss"][0], float(loss[0])) < 1e-6
    assert max_abs_rel(got["dh"], to_f64(dh, torch)) < 1e-6
    assert max_abs_rel(got["dW"], to_f64(dW, torch)) < 1e-6


def test_upstream_gradient_scales_the_shard_gradients(torch_cuda):
    inp = synth.make(0, seed=14, N=300, chunk=128)
    bounds = [(0, 3000), (3000, 8192)]
    a = _run_shards(inp, bounds, torch_cuda, chunk=128)
    b = _run_shards(inp, bounds, torch_cuda, chunk=128, g=-1.5)
    assert max_abs_rel(b["dh"], -1.5 * a["dh"]) < 1e-6
    assert max_abs_rel(b["dW"], -1.5 * a["dW"]) < 1e-6


def test_full_size_shard_of_eight(torch_cuda):
    """One GPU's share at V/8 of the 128256 vocabulary, N = 4096 tokens: the shard's
    statistics on 256 sampled rows against the shard oracle."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(1)
    V, Vs = inp.cfg.V, inp.cfg.V // 8
    a, b = 3 * Vs, 4 * Vs
    h, W, idx, p, mask = to_device(inp, torch)
    m, s, pz = kd.vocab_shard_fwd(h, W[a:b].contiguous(), idx, p, a, V, chunk=inp.cfg.chunk)
    torch.cuda.synchronize()
    rows = synth.subset_rows(inp.cfg, inp.seed, 256)
    rm, rs, rpz = oshard.shard_stats(inp.h64(rows), inp.W64()[a:b], a, inp.idx[rows],
                                     inp.p[rows])
    gm, gs, gp = (to_f64(t, torch)[rows] for t in (m, s, pz))
    _check_stats(gm, gs, gp, rm, rs, rpz)


def _check_stats(gm, gs, gp, rm, rs, rpz):
    """The shard's max, sum of exp and in-shard p.z against the oracle at the bf16
    tolerances: the max is a float32 GEMM value of exact bf16 products (relative error
    on the row maxima), the sum is compared on the oracle's scale (s * exp(m - m_ref)),
    and p.z relatively over the rows."""
    tol = TOL["bf16"]["loss"]
    errs = dict(m=max_abs_rel(gm, rm), s=max_abs_rel(gs * np.exp(gm - rm), rs),
                pz=rel_fro(gp, rpz))
    print("shard statistics:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= tol for v in errs.values()), errs


def test_index_outside_the_vocabulary_is_rejected(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(0, seed=2, N=64, chunk=64)
    inp.idx[5, 3] = inp.cfg.V + 7
    h, W, idx, p, mask = to_device(inp, torch)
    with pytest.raises(kd.KDError) as e:
        kd.vocab_shard_fwd(h, W[:1000].contiguous(), idx, p, 0, inp.cfg.V, chunk=64)
    assert e.value.code == 2


def test_bench_launch_shard_of_eight(torch_cuda):
    """The benchmark's shard launch: rows [0, V/8) of the 128256 vocabulary, N = 32768
    tokens, chunks of 16384 (eight times the unsharded chunk, the same logits-buffer
    size).  Forward statistics on 256 sampled rows; the backward, given the shard's own
    logsumexp as lse (as a one-shard vocabulary), for dh on the sampled rows and the
    shard's whole dW, all against the shard oracle."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(2)
    cfg = inp.cfg
    V, Vs, chunk = cfg.V, (cfg.V + 7) // 8, 16384
    h, W, idx, p, mask = to_device(inp, torch)
    Ws = W[:Vs].contiguous()
    m, s, pz = kd.vocab_shard_fwd(h, Ws, idx, p, 0, V, chunk=chunk)
    gm, gs, gp = (to_f64(t, torch) for t in (m, s, pz))
    del m, s, pz
    H, Wsh = inp.h64(), inp.W64()[:Vs]
    rows = synth.subset_rows(cfg, inp.seed, 256)
    rm, rs, rpz = oshard.shard_stats(H, Wsh, 0, inp.idx, inp.p, block_rows=1024)
    _check_stats(gm[rows], gs[rows], gp[rows], rm[rows], rs[rows], rpz[rows])
    lse32 = (rm + np.log(rs)).astype(np.float32)
    dh_rows, dW = oshard.shard_backward(H, Wsh, 0, inp.idx, inp.p, lse32.astype(np.float64),
                                        inp.mask, block_rows=1024, rows=rows)
    dhp, dWp = kd.vocab_shard_bwd(h, Ws, idx, p, torch.from_numpy(lse32).cuda(), 0, V, None,
                                  mask, chunk=chunk)
    torch.cuda.synchronize()
    e_dh = rel_fro(to_f64(dhp, torch)[rows], dh_rows)
    e_dW = rel_fro(to_f64(dWp, torch), dW)
    print(f"shard of eight at the bench launch: dh rows {e_dh:.2e}, dW {e_dW:.2e}", flush=True)
    assert e_dh <= TOL["bf16"]["grad"] and e_dW <= TOL["bf16"]["grad"]
