"""Helpers shared by the GPU tests: move seeded inputs to the device, run the HIP path
through the C ABI, and compare against the oracle with the stated metrics."""
import numpy as np

import synth

# Tolerances: fp32 workloads 1e-5 relative on the loss and 1e-4 max-abs-relative on
# dh and dW; bf16 workloads 2e-3 relative on the loss and 3e-2 relative Frobenius on
# dh and dW.  The gathered logits (zg) and logsumexp are compared with the same
# metric as the gradients of that precision.
TOL = {
    "f32": dict(loss=1e-5, grad=1e-4, metric="max_abs_rel"),
    "bf16": dict(loss=2e-3, grad=3e-2, metric="rel_fro"),
}

# The gathered logits zg[n, k] = z[n, idx[n, k]] are a float32 MFMA sum of the d products
# h[n, j] * W[v, j], exact for bf16 inputs (8-bit significands, so every product fits a
# float32) and rounded once each for float32 inputs; the oracle sums the same products in
# float64.  Float32 accumulation of d terms errs by about sqrt(d) * 2^-24 of the partial
# sums' size: at d = 3072 with |z| ~ 2, about 1e-6 of |z|.  1e-5 (relative Frobenius over
# rows, or max-abs-relative on small cases) leaves a tenfold margin and is far below what a
# wrong accumulator, row or column would give (errors of the size of z itself).
ZG_TOL = 1e-5


def rel(a, b):
    return abs(float(a) - float(b)) / max(abs(float(b)), 1e-300)


def max_abs_rel(g, o):
    g = np.asarray(g, np.float64); o = np.asarray(o, np.float64)
    den = np.abs(o).max()
    return float(np.abs(g - o).max() / den) if den > 0 else float(np.abs(g).max())


def rel_fro(g, o):
    g = np.asarray(g, np.float64); o = np.asarray(o, np.float64)
    den = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / den) if den > 0 else float(np.linalg.norm(g))


def grad_err(dtype, g, o):
    return max_abs_rel(g, o) if TOL[dtype]["metric"] == "max_abs_rel" else rel_fro(g, o)


def to_device(inp: synth.Inputs, torch):
    dev = "cuda"
    if inp.cfg.dtype == "bf16":
        h = torch.from_numpy(inp.h.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        h = torch.from_numpy(inp.h).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    idx = torch.from_numpy(inp.idx).to(dev)
    p = torch.from_numpy(inp.p).to(dev)
    mask = torch.from_numpy(inp.mask).to(dev)
    return h, W, idx, p, mask


def to_f64(t, torch):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_raw(inp: synth.Inputs, torch, chunk=None, rows=True, use_mask=True, **kw):
    """Outputs of the HIP path as torch tensors on the device (``kw`` goes to fwd_bwd)."""
    import output_head_kl_amd as kd
    h, W, idx, p, mask = to_device(inp, torch)
    out = kd.fwd_bwd(h, W, idx, p, mask if use_mask else None,
                     chunk=chunk or inp.cfg.chunk, rows=rows, **kw)
    torch.cuda.synchronize()
    del h, W, idx, p, mask
    names = ["loss", "dh", "dW", "row_loss", "row_lse", "zg"][:len(out)]
    return dict(zip(names, out))


def run(inp: synth.Inputs, torch, chunk=None, rows=True, use_mask=True, **kw):
    """Outputs of the HIP path as float64 numpy arrays."""
    return {k: to_f64(v, torch)
            for k, v in run_raw(inp, torch, chunk, rows, use_mask, **kw).items()}
