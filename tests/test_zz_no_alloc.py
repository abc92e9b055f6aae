"""The allocation-free teacher top-K producer (kd_teacher_topk_noalloc) through the C ABI
against the allocating call (kd_teacher_topk) on the same logits: indices, probabilities
and logsumexp bit for bit, on two calls in a row (the second smaller, so the shared
scratch carries the first call's state into it), and the invalid-row error followed by a
good call (the flag is cleared at the start of every call)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _alloc_call(kd, torch, x, dt, K):
    N, V = x.shape
    idx = torch.empty((N, K), dtype=torch.int32, device="cuda")
    p = torch.empty((N, K), dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    rc = kd._lib().kd_teacher_topk(x.data_ptr(), dt, N, V, K, idx.data_ptr(), p.data_ptr(),
                                   lse.data_ptr(), ws.data_ptr(), 256,
                                   torch.cuda.current_stream().cuda_stream)
    return rc, idx, p, lse


def _noalloc_call(kd, torch, x, dt, K):
    N, V = x.shape
    idx = torch.full((N, K), -7, dtype=torch.int32, device="cuda")
    p = torch.full((N, K), -7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((N,), -7.0, dtype=torch.float32, device="cuda")
    rc = kd._lib().kd_teacher_topk_noalloc(x.data_ptr(), dt, N, V, K, idx.data_ptr(),
                                           p.data_ptr(), lse.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    return rc, idx, p, lse


def _bits(t):
    return t.contiguous().cpu().numpy().view(np.uint8)


def test_noalloc_matches_allocating_call_on_two_calls(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    cases = [("bf16", 2048, 128256, 100), ("f32", 300, 5003, 37)]   # the second is smaller
    for dtype, N, V, K in cases:
        print(f"noalloc top-K: dtype={dtype} N={N} V={V} K={K}", flush=True)
        bits = synth.make_teacher_logits(N, V, seed=synth.BASE_SEED + 40 + N, threads=8)
        x32 = synth.bf16_bits_to_f32(bits)
        if dtype == "bf16":
            x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
            dt = kd.KD_BF16
        else:
            x = torch.from_numpy(np.ascontiguousarray(x32)).cuda()
            dt = kd.KD_F32
        a = _alloc_call(kd, torch, x, dt, K)
        b = _noalloc_call(kd, torch, x, dt, K)
        torch.cuda.synchronize()
        assert a[0] == 0 and b[0] == 0, (a[0], b[0], kd._lib().kd_last_error())
        for ta, tb in zip(a[1:], b[1:]):
            assert np.array_equal(_bits(ta), _bits(tb))


def test_noalloc_rejects_a_bad_row_then_recovers(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    x = torch.randn((64, 3000), device="cuda")
    x[17, 5] = float("nan")
    rc, *_ = _noalloc_call(kd, torch, x, kd.KD_F32, 10)
    torch.cuda.synchronize()
    assert rc == 2, kd._lib().kd_last_error()
    x[17, 5] = 0.0
    rc, idx, p, lse = _noalloc_call(kd, torch, x, kd.KD_F32, 10)
    ra = _alloc_call(kd, torch, x, kd.KD_F32, 10)
    torch.cuda.synchronize()
    assert rc == 0 and ra[0] == 0
    assert torch.equal(idx, ra[1]) and torch.equal(p, ra[2]) and torch.equal(lse, ra[3])


def test_noalloc_argument_errors_and_empty_batch(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    lib = kd._lib()
    x = torch.randn((4, 50), device="cuda")
    out_i = torch.empty((4, 8), dtype=torch.int32, device="cuda")
    out_p = torch.empty((4, 8), device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.kd_teacher_topk_noalloc(x.data_ptr(), 0, 4, 50, 51, out_i.data_ptr(),
                                       out_p.data_ptr(), None, s) == 1      # K > V
    assert lib.kd_teacher_topk_noalloc(x.data_ptr(), 0, 4, 50, 300, out_i.data_ptr(),
                                       out_p.data_ptr(), None, s) != 0      # K above 256
    assert lib.kd_teacher_topk_noalloc(None, 0, 0, 50, 8, None, None, None, s) == 0
