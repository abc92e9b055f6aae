"""The forward and backward halves (kd_chunked_kl_fwd / kd_chunked_kl_bwd) through the C
ABI: with an upstream gradient of 1 they reproduce the fused call's forward outputs bit
for bit and its gradients to rounding (the backward half recomputes the logits; the
fused call keeps each chunk's exp(z - max) from its forward), an upstream gradient g
scales dh and dW, the autograd wrapper gives the oracle's gradients, and the edge cases
behave as in the fused call."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, grad_err, max_abs_rel, rel, to_device, to_f64

pytestmark = pytest.mark.gpu


def _split(inp, torch, chunk=None, g=None, use_mask=True):
    import output_head_kl_amd as kd
    h, W, idx, p, mask = to_device(inp, torch)
    m = mask if use_mask else None
    chunk = chunk or inp.cfg.chunk
    loss, row_lse, row_loss, zg = kd.fwd(h, W, idx, p, m, chunk=chunk, rows=True)
    gt = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    dh, dW = kd.bwd(h, W, idx, p, row_lse, gt, m, chunk=chunk)
    torch.cuda.synchronize()
    return dict(loss=loss, row_lse=row_lse, row_loss=row_loss, zg=zg, dh=dh, dW=dW)


def _fused(inp, torch, chunk=None, use_mask=True):
    import output_head_kl_amd as kd
    h, W, idx, p, mask = to_device(inp, torch)
    out = kd.fwd_bwd(h, W, idx, p, mask if use_mask else None, chunk=chunk or inp.cfg.chunk,
                     rows=True)
    torch.cuda.synchronize()
    return dict(zip(["loss", "dh", "dW", "row_loss", "row_lse", "zg"], out))


def _bits(t, torch):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _same_as_fused(a, b, dtype, torch, fwd_keys):
    for k in fwd_keys:
        assert np.array_equal(_bits(a[k], torch), _bits(b[k], torch)), k
    for k in ["dh", "dW"]:
        ga, gb = to_f64(a[k], torch), to_f64(b[k], torch)
        assert grad_err(dtype, ga, gb) <= TOL[dtype]["grad"], k
    # rows of masked tokens are exactly zero in both
    za, zb = np.all(to_f64(a["dh"], torch) == 0, axis=1), np.all(to_f64(b["dh"], torch) == 0, axis=1)
    assert np.array_equal(za, zb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_matches_fused(torch_cuda, dtype):
    """Ragged shapes (V, d, N off the tile grid, partial last chunk), masked rows and a
    repeated index: fwd + bwd(g = 1) give the fused call's forward outputs bit for bit
    and its gradients within the gradient tolerance."""
    torch = torch_cuda
    inp = synth.make(1, seed=91, N=700, d=264, V=3001, K=7, chunk=300, dtype=dtype)
    inp.mask[[0, 5, 299, 300, 699]] = 0
    inp.idx[3, 1] = inp.idx[3, 0]
    a, b = _split(inp, torch), _fused(inp, torch)
    _same_as_fused(a, b, dtype, torch, ["loss", "row_lse", "row_loss", "zg"])


def test_split_matches_fused_full_size(torch_cuda):
    """The 4096-token, V = 128256 workload in the benchmark's launch configuration."""
    torch = torch_cuda
    inp = synth.make(1)
    a, b = _split(inp, torch), _fused(inp, torch)
    _same_as_fused(a, b, "bf16", torch, ["loss", "row_lse"])


def test_split_against_oracle_with_upstream_gradient(torch_cuda):
    torch = torch_cuda
    g = -2.5
    inp = synth.make(0, seed=17, N=300, chunk=128)
    inp.mask[[1, 2, 250]] = 0
    got = {k: to_f64(v, torch) for k, v in _split(inp, torch, g=g).items()}
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL["f32"]
    assert rel(got["loss"][0], ref["loss"]) <= tol["loss"]
    assert max_abs_rel(got["row_lse"], ref["row_lse"]) <= tol["loss"]
    assert grad_err("f32", got["dh"], g * ref["dh"]) <= tol["grad"]
    assert grad_err("f32", got["dW"], g * ref["dW"]) <= tol["grad"]
    assert np.all(got["dh"][inp.mask == 0] == 0.0)


def test_upstream_gradient_zero_gives_zero_gradients(torch_cuda):
    torch = torch_cuda
    inp = synth.make(0, seed=3, N=200, chunk=64)
    got = _split(inp, torch, g=0.0)
    assert float(got["dh"].abs().max()) == 0.0 and float(got["dW"].abs().max()) == 0.0


def test_autograd_wrapper_matches_oracle(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(1, seed=23, N=500, d=256, V=5000, K=16, chunk=192, dtype="bf16")
    h, W, idx, p, mask = to_device(inp, torch)
    h = h.clone().requires_grad_(True)
    W = W.clone().requires_grad_(True)
    loss = kd.chunked_kl_loss(h, W, idx, p, mask, chunk=192)
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL["bf16"]
    assert loss.dim() == 0
    assert rel(float(loss.detach()), ref["loss"]) <= tol["loss"]
    assert h.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    assert grad_err("bf16", to_f64(h.grad, torch), 3.0 * ref["dh"]) <= tol["grad"]
    assert grad_err("bf16", to_f64(W.grad, torch), 3.0 * ref["dW"]) <= tol["grad"]


def test_split_all_masked_and_empty(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(0, seed=8, N=130, chunk=64)
    inp.mask[:] = 0
    got = _split(inp, torch)
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    assert float(got["loss"][0]) == 0.0
    assert float(got["dh"].abs().max()) == 0.0 and float(got["dW"].abs().max()) == 0.0
    # the per-row logsumexp is still produced (the backward would read it)
    assert max_abs_rel(to_f64(got["row_lse"], torch), ref["row_lse"]) <= TOL["f32"]["loss"]
    # N = 0
    dev = "cuda"
    h = torch.zeros((0, 16), device=dev)
    W = torch.randn((50, 16), device=dev)
    idx = torch.zeros((0, 3), dtype=torch.int32, device=dev)
    p = torch.zeros((0, 3), dtype=torch.float32, device=dev)
    loss, row_lse = kd.fwd(h, W, idx, p, chunk=8)
    dh, dW = kd.bwd(h, W, idx, p, row_lse, None, chunk=8)
    torch.cuda.synchronize()
    assert float(loss[0]) == 0.0 and dh.shape == (0, 16) and float(dW.abs().max()) == 0.0


def test_split_rejects_invalid_entries_without_writing(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(0, seed=4, N=100, chunk=64)
    inp.idx[7, 2] = inp.cfg.V
    h, W, idx, p, mask = to_device(inp, torch)
    with pytest.raises(kd.KDError) as e:
        kd.fwd(h, W, idx, p, mask, chunk=64)
    assert e.value.code == 2
    lse = torch.zeros(inp.cfg.N, dtype=torch.float32, device="cuda")
    dh = torch.full((inp.cfg.N, inp.cfg.d), 7.0, device="cuda")
    dW = torch.full((inp.cfg.V, inp.cfg.d), 7.0, device="cuda")
    ws = torch.empty(kd.workspace_bytes(inp.cfg.N, inp.cfg.d, inp.cfg.V, inp.cfg.K, 64, kd.KD_F32),
                     dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    rc = kd._lib().kd_chunked_kl_bwd(h.data_ptr(), W.data_ptr(), kd.KD_F32, idx.data_ptr(),
                                     p.data_ptr(), mask.data_ptr(), inp.cfg.N, inp.cfg.d,
                                     inp.cfg.V, inp.cfg.K, 64, lse.data_ptr(), g.data_ptr(),
                                     dh.data_ptr(), dW.data_ptr(), ws.data_ptr(), ws.numel(),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 2
    assert float(dh.min()) == 7.0 and float(dW.max()) == 7.0


@pytest.mark.parametrize("dtype,g", [("bf16", 3.0), ("f32", -2.5)])
def test_fused_autograd_mode_matches_oracle(torch_cuda, dtype, g):
    """chunked_kl_loss(mode='fused'): the forward runs the one-call loss and gradients
    (dh kept in float32), the backward applies the upstream gradient g on the device
    (kd_scale_grads); the gradients are g times the oracle's, and agree with the
    recompute mode's."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(1, seed=29, N=500, d=256, V=5000, K=16, chunk=192, dtype=dtype)
    inp.mask[[0, 77, 499]] = 0
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL[dtype]
    grads = {}
    for mode in ("fused", "recompute"):
        h, W, idx, p, mask = to_device(inp, torch)
        h = h.clone().requires_grad_(True)
        W = W.clone().requires_grad_(True)
        loss = kd.chunked_kl_loss(h, W, idx, p, mask, chunk=192, mode=mode)
        (g * loss).backward()
        torch.cuda.synchronize()
        assert loss.dim() == 0 and rel(float(loss.detach()), ref["loss"]) <= tol["loss"]
        assert h.grad.dtype == h.dtype and W.grad.dtype == W.dtype
        grads[mode] = (to_f64(h.grad, torch), to_f64(W.grad, torch))
        errs = dict(dh=grad_err(dtype, grads[mode][0], g * ref["dh"]),
                    dW=grad_err(dtype, grads[mode][1], g * ref["dW"]))
        print(dtype, mode, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        assert errs["dh"] <= tol["grad"] and errs["dW"] <= tol["grad"], errs
        assert np.all(grads[mode][0][inp.mask == 0] == 0.0)
    assert grad_err(dtype, grads["fused"][0], grads["recompute"][0]) <= tol["grad"]
    assert grad_err(dtype, grads["fused"][1], grads["recompute"][1]) <= tol["grad"]


def test_fused_autograd_mode_with_unit_gradient_is_the_one_call(torch_cuda):
    """With g = 1 the backward's product is exact: dh (rounded once from the same float32
    sums) equals the one-call kd_chunked_kl_fwd_bwd output bit for bit, and W's gradient
    is that call's float32 dW as autograd casts it to W's dtype."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    inp = synth.make(1, seed=30, N=700, d=264, V=3001, K=7, chunk=300, dtype="bf16")
    inp.mask[[4, 300]] = 0
    h, W, idx, p, mask = to_device(inp, torch)
    loss1, dh1, dW1 = kd.fwd_bwd(h, W, idx, p, mask, chunk=300)
    hg = h.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = kd.chunked_kl_loss(hg, Wg, idx, p, mask, chunk=300)
    loss.backward()
    torch.cuda.synchronize()
    assert float(loss.detach()) == float(loss1[0])
    assert np.array_equal(_bits(hg.grad, torch), _bits(dh1, torch))
    assert np.array_equal(_bits(Wg.grad, torch), _bits(dW1.to(torch.bfloat16), torch))


def test_scale_grads_rounds_once(torch_cuda):
    """kd_scale_grads: dh = g * dh_f32 rounded once to bf16 (compared with torch's own
    float32 product and bf16 rounding), dW scaled in place, and a dW left untouched for
    g = 1."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    gen = torch.Generator(device="cuda").manual_seed(5)
    dh32 = torch.randn((37, 24), device="cuda", generator=gen)
    dW = torch.randn((19, 24), device="cuda", generator=gen)
    dW0 = dW.clone()
    g = torch.tensor([-0.3], device="cuda")
    dh, dW_out = kd.scale_grads(g, dh32, dW, torch.bfloat16)
    torch.cuda.synchronize()
    assert dW_out.data_ptr() == dW.data_ptr()
    assert torch.equal(dh, (dh32 * g).to(torch.bfloat16))
    assert torch.equal(dW, dW0 * g)
    one = torch.ones(1, device="cuda")
    dh, _ = kd.scale_grads(one, dh32, dW, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dh, dh32) and torch.equal(dW, dW0 * g)
