"""Device memory of the fused call (peak memory linear in the sequence length, only
transient logits: codewithpapers.app abstract; legiblepapers.com summary, Q4).

* Peak memory of one call is a + b*N: with the smallest workspace for every N, and with
  the default workspace once N fills its dW group (the workspace is constant from there);
  b is what the per-token tensors need (h and dh in bf16, the teacher's indices and
  probabilities, the mask).
* The library allocates nothing of its own: across a call the device's free memory drops
  by no more than torch's pool grows (every buffer comes from torch).
* No allocation is the size of the batch's logits (N x V bf16): torch's pool, emptied
  before the call, holds no segment that large afterwards.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

d, V, K, CHUNK = 1024, 32768, 100, 1024
PER_TOKEN = 2 * d + 2 * d + 8 * K + 1          # h, dh (bf16), idx + p, mask


def _warm(torch, kd):
    """One small call first, so that loading the library's code onto the device is not
    counted against the calls measured."""
    h = torch.zeros((64, d), device="cuda", dtype=torch.bfloat16)
    W = torch.zeros((V, d), device="cuda", dtype=torch.bfloat16)
    idx = torch.zeros((64, K), device="cuda", dtype=torch.int32)
    p = torch.full((64, K), 1.0 / K, device="cuda")
    kd.fwd_bwd(h, W, idx, p, None, chunk=CHUNK)
    torch.cuda.synchronize()


def _peak_of_call(torch, kd, N, group):
    g = torch.Generator(device="cuda").manual_seed(N)
    W = torch.randn(V, d, device="cuda", generator=g, dtype=torch.bfloat16) * (2.0 / d ** 0.5)
    h = torch.randn(N, d, device="cuda", generator=g, dtype=torch.bfloat16)
    idx = torch.randint(0, V, (N, K), device="cuda", generator=g, dtype=torch.int32)
    p = torch.rand(N, K, device="cuda", generator=g) / K
    mask = torch.ones(N, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    free0, _ = torch.cuda.mem_get_info()
    res0 = torch.cuda.memory_reserved()
    out = kd.fwd_bwd(h, W, idx, p, mask, chunk=CHUNK, dw_group_tokens=group)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    res1 = torch.cuda.memory_reserved()
    peak = torch.cuda.max_memory_allocated()
    largest = max((seg["total_size"] for seg in torch.cuda.memory_snapshot()), default=0)
    loss = float(out[0].item())
    del out, W, h, idx, p, mask
    torch.cuda.empty_cache()
    return dict(peak=peak, free_drop=free0 - free1, pool_growth=res1 - res0, largest=largest,
                loss=loss)


def _fit(Ns, peaks):
    x, y = np.asarray(Ns, np.float64), np.asarray(peaks, np.float64)
    b, a = np.polyfit(x, y, 1)
    return a, b, float(np.abs(y - (a + b * x)).max())


@pytest.mark.parametrize("group", [0, None])
def test_peak_memory_is_linear_in_tokens(torch_cuda, group):
    import output_head_kl_amd as kd
    torch = torch_cuda
    _warm(torch, kd)
    # the default dW group (16384 tokens) holds the whole batch below that: fit past it
    Ns = [4096, 8192, 16384, 32768] if group == 0 else [16384, 24576, 32768, 49152]
    runs = {N: _peak_of_call(torch, kd, N, group) for N in Ns}
    a, b, resid = _fit(Ns, [runs[N]["peak"] for N in Ns])
    print(f"dw group {group}: peak = {a / 2**30:.3f} GiB + {b:.1f} B/token "
          f"(expected {PER_TOKEN}), max residual {resid / 2**20:.2f} MiB", flush=True)
    for N, r in runs.items():
        print(f"  N={N}: peak {r['peak'] / 2**30:.3f} GiB, free drop {r['free_drop'] / 2**20:.1f} "
              f"MiB, pool growth {r['pool_growth'] / 2**20:.1f} MiB, largest segment "
              f"{r['largest'] / 2**20:.1f} MiB, N*V*2 {N * V * 2 / 2**20:.0f} MiB", flush=True)
        assert np.isfinite(r["loss"])
        # nothing outside torch's pool (2 MiB of slack for the runtime's own bookkeeping)
        assert r["free_drop"] <= r["pool_growth"] + (2 << 20), (N, r)
    # linear with the per-token tensors' bytes as slope (the pool rounds each tensor up)
    assert abs(b - PER_TOKEN) <= 0.01 * PER_TOKEN, b
    assert resid <= 4 << 20, resid


def test_no_allocation_of_the_batch_logits_size(torch_cuda):
    """With the smallest workspace no buffer reaches N x V bf16 once N >= 8 chunks; with the
    default workspace (dW group of 16384 tokens) once N is past the group."""
    import output_head_kl_amd as kd
    torch = torch_cuda
    _warm(torch, kd)
    for N, group in [(8 * CHUNK, 0), (32 * CHUNK, 0), (32768, None), (65536, None)]:
        r = _peak_of_call(torch, kd, N, group)
        ws = kd.workspace_bytes(N, d, V, K, CHUNK, dw_group_tokens=group)
        print(f"N={N} group={group}: workspace {ws / 2**20:.0f} MiB, largest segment "
              f"{r['largest'] / 2**20:.0f} MiB, N*V*2 {N * V * 2 / 2**20:.0f} MiB", flush=True)
        assert ws < N * V * 2
        assert r["largest"] < N * V * 2
