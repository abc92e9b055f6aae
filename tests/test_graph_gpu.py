"""The one-call loss without its host synchronisation (kd_chunked_kl_fwd_bwd_async):

* equal bit for bit to kd_chunked_kl_fwd_bwd, with per-row outputs and a ragged last
  chunk, in bf16 and fp32;
* recorded once into a HIP graph (torch.cuda.graph) and replayed for three new contents
  of the same input buffers, with eager work of the program's own and synchronisations
  between the replays: every replay equals the synchronising call on those contents bit
  for bit;
* an invalid teacher entry (index V, an index far past the vocabulary, a negative index,
  a NaN probability) raises the status word without a fault, and a valid call on the same
  buffers afterwards is right again;
* a batch whose mask counts no token gives loss 0, dh 0, dW 0 and status 0."""
import numpy as np
import pytest

import output_head_kl_amd as kd
import synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu
KD_E_INDEX = 2
KEYS = ("loss", "dh", "dW", "row_loss", "row_lse", "zg")


def _bits(t, torch):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _alloc(torch, h, W, idx, chunk):
    N, d = h.shape
    V, K = W.shape[0], idx.shape[1]
    dt = kd.KD_BF16 if h.dtype == torch.bfloat16 else kd.KD_F32
    ws = torch.empty(kd.workspace_bytes(N, d, V, K, chunk, dt), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = dict(loss=torch.empty(1, **f32), dh=torch.empty_like(h), dW=torch.empty((V, d), **f32),
               row_loss=torch.empty(N, **f32), row_lse=torch.empty(N, **f32),
               zg=torch.empty((N, K), **f32),
               status=torch.full((1,), -1, dtype=torch.int32, device="cuda"))
    return ws, out


def _async(h, W, idx, p, mask, ws, out, chunk):
    kd.fwd_bwd_async(h, W, idx, p, mask, out["loss"], out["dh"], out["dW"], out["status"], ws,
                     chunk=chunk, row_loss=out["row_loss"], row_lse=out["row_lse"],
                     zg=out["zg"])


def _sync(h, W, idx, p, mask, chunk):
    return dict(zip(KEYS, kd.fwd_bwd(h, W, idx, p, mask, chunk=chunk, rows=True)))


def _same(a, b, torch):
    for k in KEYS:
        assert np.array_equal(_bits(a[k], torch), _bits(b[k], torch)), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_async_equals_the_synchronising_call(torch_cuda, dtype):
    torch = torch_cuda
    inp = synth.make(1, seed=71, N=700, d=264, V=3001, K=7, chunk=300, dtype=dtype)
    inp.mask[[0, 299, 699]] = 0
    h, W, idx, p, mask = to_device(inp, torch)
    ws, out = _alloc(torch, h, W, idx, 300)
    print(f"async {dtype} N=700 d=264 V=3001 chunk=300", flush=True)
    _async(h, W, idx, p, mask, ws, out, 300)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    _same(out, _sync(h, W, idx, p, mask, 300), torch)


def test_graph_replays_match_the_synchronising_call(torch_cuda):
    torch = torch_cuda
    N, d, V, K, C = 600, 136, 2500, 9, 256     # chunks of 256, 256 and 88 tokens
    base = synth.make(1, seed=72, N=N, d=d, V=V, K=K, chunk=C)
    h, W, idx, p, mask = to_device(base, torch)
    ws, out = _alloc(torch, h, W, idx, C)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # a first call off the recording
        _async(h, W, idx, p, mask, ws, out, C)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    print("recording the graph", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _async(h, W, idx, p, mask, ws, out, C)
    torch.cuda.synchronize()
    for rep in range(3):
        new = synth.make(1, seed=80 + rep, N=N, d=d, V=V, K=K, chunk=C)
        new.mask[[rep, 300 + rep]] = 0
        for dst, src in zip((h, W, idx, p, mask), to_device(new, torch)):
            dst.copy_(src)
        a = torch.randn(512, 512, device="cuda")
        float((a @ a).sum())                 # eager work and a synchronisation between replays
        print(f"replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        _same(out, _sync(h, W, idx, p, mask, C), torch)


@pytest.mark.parametrize("bad", ["index_V", "index_far", "index_negative", "nan_p"])
def test_invalid_entry_sets_the_status_without_a_fault(torch_cuda, bad):
    torch = torch_cuda
    inp = synth.make(1, seed=73, N=300, d=72, V=1000, K=5, chunk=128)
    h, W, idx, p, mask = to_device(inp, torch)
    ws, out = _alloc(torch, h, W, idx, 128)
    if bad == "index_V":
        idx[7, 2] = 1000
    elif bad == "index_far":
        idx[7, 2] = 2**30
    elif bad == "index_negative":
        idx[7, 2] = -5
    else:
        p[7, 2] = float("nan")
    print(f"async with a bad entry: {bad}", flush=True)
    _async(h, W, idx, p, mask, ws, out, 128)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == KD_E_INDEX
    idx.copy_(torch.from_numpy(inp.idx).cuda())
    p.copy_(torch.from_numpy(inp.p).cuda())
    _async(h, W, idx, p, mask, ws, out, 128)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    _same(out, _sync(h, W, idx, p, mask, 128), torch)


def test_no_counted_token(torch_cuda):
    torch = torch_cuda
    inp = synth.make(1, seed=74, N=300, d=72, V=1000, K=5, chunk=128)
    inp.mask[:] = 0
    h, W, idx, p, mask = to_device(inp, torch)
    ws, out = _alloc(torch, h, W, idx, 128)
    _async(h, W, idx, p, mask, ws, out, 128)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    assert float(out["loss"].item()) == 0.0
    assert bool((out["dh"] == 0).all()) and bool((out["dW"] == 0).all())
    ref = _sync(h, W, idx, p, mask, 128)
    for k in ("row_loss", "row_lse", "zg"):
        assert np.array_equal(_bits(out[k], torch), _bits(ref[k], torch)), k
