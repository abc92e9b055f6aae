"""The C-ABI library loads, exports every declared symbol, and rejects bad calls on the
host before touching a device (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

import output_head_kl_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdkl.h")

OK, E_ARG, E_INDEX, E_WORKSPACE, E_UNSUPPORTED, E_HIP = range(6)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kd.library_path()):
        pytest.fail("libkdkl.so is not built (run __graft_entry__.build())")
    return kd._lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"kd_workspace_bytes", "kd_chunked_kl_fwd_bwd", "kd_last_error"} <= set(names)
    raw = ctypes.CDLL(kd.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in kdkl.h but not exported"


def test_version_and_profile_classes(lib):
    assert lib.kd_version() == 5
    names = kd.profile_classes()
    assert "fwd_gemm_lse" in names and "dw_gemm" in names and len(names) == len(set(names))


def test_workspace_is_bounded_and_constant_beyond_one_dw_group(lib):
    """The workspace holds one chunk's dz and a dW group of at most 16384 tokens (never
    more chunks than the batch has): constant in N from there on, with no N x V term."""
    a = kd.workspace_bytes(32768, 3072, 128256, 100, 2048)
    b = kd.workspace_bytes(262144, 3072, 128256, 100, 2048)
    c = kd.workspace_bytes(16384, 3072, 128256, 100, 2048)
    assert a == b == c
    assert a % 256 == 0
    # one chunk's dz, the token-contiguous dz of a 16384-token dW group (bf16) and W^T
    # dominate
    dz, dzt, wt = 2048 * 128256 * 2, 16384 * 128256 * 2, 128256 * 3072 * 2
    assert dz + dzt + wt < a < dz + dzt + wt + 600_000_000
    # smaller batches get a smaller dW group: two 2048-token chunks at N = 4096
    d = kd.workspace_bytes(4096, 3072, 128256, 100, 2048)
    assert d == a - (16384 - 4096) * 128256 * 2 - (16384 - 4096) * 3072 * 2
    small = kd.workspace_bytes(100, 3072, 128256, 100, 2048)
    assert small < d < a
    # sizes never decrease with N
    sizes = [kd.workspace_bytes(n, 3072, 128256, 100, 2048) for n in (1, 2048, 2049, 8192, 20000)]
    assert sizes == sorted(sizes)


def test_workspace_for_a_smaller_dw_group(lib):
    """Each token of the dW group costs (V_pad + d) * 2 bytes; group 0 (one chunk) keeps
    no more than one chunk's logits anywhere, and 16384 is the default."""
    args = (32768, 3072, 128256, 100, 2048)
    full = kd.workspace_bytes(*args)
    assert kd.workspace_bytes(*args, dw_group_tokens=16384) == full
    assert kd.workspace_bytes(*args, dw_group_tokens=1 << 30) == full
    one = kd.workspace_bytes(*args, dw_group_tokens=0)
    assert kd.workspace_bytes(*args, dw_group_tokens=2047) == one
    assert kd.workspace_bytes(*args, dw_group_tokens=2048) == one
    per_token = (128256 + 3072) * 2
    for g in (2, 3, 5, 8):
        assert kd.workspace_bytes(*args, dw_group_tokens=g * 2048 + 100) == one + (g - 1) * 2048 * per_token
    assert full == one + 7 * 2048 * per_token
    dz, wt = 2048 * 128256 * 2, 128256 * 3072 * 2
    assert 2 * dz + wt < one < 2 * dz + wt + 600_000_000
    # fp32 always accumulates dW chunk by chunk
    assert kd.workspace_bytes(*args, kd.KD_F32, 0) == kd.workspace_bytes(*args, kd.KD_F32)
    out = ctypes.c_size_t(0)
    assert lib.kd_workspace_bytes_group(*args, 1, -1, ctypes.byref(out)) == E_ARG


@pytest.mark.parametrize("args,code", [
    ((10, 12, 100, 4, 8, 1), E_UNSUPPORTED),     # d not a multiple of 8
    ((10, 16, 100, 0, 8, 1), E_ARG),             # K = 0
    ((10, 16, 100, 4, 0, 1), E_ARG),             # chunk = 0
    ((10, 16, 0, 4, 8, 1), E_ARG),               # V = 0
    ((-1, 16, 100, 4, 8, 1), E_ARG),             # N < 0
    ((10, 16, 100, 4, 8, 7), E_ARG),             # unknown dtype
    ((10, 16, 100, 70000, 8, 1), E_UNSUPPORTED),  # K too large
    ((1 << 23, 16, 100, 4, 1 << 23, 1), E_UNSUPPORTED),   # 2^23 rows in one chunk
    ((1 << 22, 16, 100, 1024, 1 << 22, 1), E_UNSUPPORTED),  # 2^32 teacher entries per chunk
])
def test_workspace_query_rejects_bad_sizes(lib, args, code):
    out = ctypes.c_size_t(0)
    assert lib.kd_workspace_bytes(*args, ctypes.byref(out)) == code
    assert lib.kd_last_error()


def _call(lib, **kw):
    """Call the entry point with fake but aligned device addresses; every case below must
    be rejected by host checks before any device work."""
    base = dict(h=0x100000, W=0x200000, dtype=1, idx=0x300000, p=0x400000, mask=None, N=64,
                d=64, V=1000, K=4, chunk=32, loss=0x500000, dh=0x600000, dW=0x700000,
                row_loss=None, row_lse=None, zg=None, ws=0x800000, wsb=1 << 40, stream=None)
    base.update(kw)
    b = base
    return lib.kd_chunked_kl_fwd_bwd(b["h"], b["W"], b["dtype"], b["idx"], b["p"], b["mask"],
                                     b["N"], b["d"], b["V"], b["K"], b["chunk"], b["loss"],
                                     b["dh"], b["dW"], b["row_loss"], b["row_lse"], b["zg"],
                                     b["ws"], b["wsb"], b["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), E_ARG),
    (dict(h=None), E_ARG),
    (dict(idx=None), E_ARG),
    (dict(dW=None), E_ARG),
    (dict(loss=None), E_ARG),
    (dict(ws=None), E_ARG),
    (dict(h=0x100008), E_ARG),       # h not 16-byte aligned
    (dict(dW=0x700004), E_ARG),
    (dict(ws=0x800010), E_ARG),      # workspace not 256-byte aligned
    (dict(p=0x400002), E_ARG),
    (dict(d=60), E_UNSUPPORTED),
    (dict(chunk=0), E_ARG),
    (dict(wsb=1000), E_WORKSPACE),
    (dict(N=(1 << 22) + 1, chunk=1 << 30), E_UNSUPPORTED),  # one chunk above 2^22 rows
])
def test_entry_point_rejects_bad_calls_on_host(lib, kw, code):
    assert _call(lib, **kw) == code
    assert lib.kd_last_error()


def test_rows_per_chunk_limit_is_on_the_chunk_not_the_batch(lib):
    """A chunk above the batch means one chunk of N rows: the 2^22-row limit applies to
    min(chunk, N), so a huge chunk over a small batch and a huge batch in small chunks
    are both accepted."""
    out = ctypes.c_size_t(0)
    assert lib.kd_workspace_bytes(1000, 16, 100, 4, 1 << 40, 1, ctypes.byref(out)) == OK
    assert lib.kd_workspace_bytes(1 << 30, 16, 100, 4, 4096, 1, ctypes.byref(out)) == OK
    assert lib.kd_workspace_bytes(1 << 22, 16, 100, 4, 1 << 22, 1, ctypes.byref(out)) == OK


def test_more_teacher_entries_than_vocabulary_is_accepted(lib):
    """K > V is valid: a row then repeats indices, whose probabilities add up in the
    gradient (scatter-add) while the gather reads each entry; only the range of each
    index is checked (on the device)."""
    out = ctypes.c_size_t(0)
    assert lib.kd_workspace_bytes(64, 64, 10, 40, 32, 1, ctypes.byref(out)) == OK
    assert _call(lib, V=10, K=40, wsb=1000) == E_WORKSPACE   # passes every size check


def test_workspace_too_small_reports_needed_size(lib):
    """Below the one-chunk dW group the call fails; the message gives that size."""
    need = kd.workspace_bytes(64, 64, 1000, 4, 32, dw_group_tokens=0)
    assert need < kd.workspace_bytes(64, 64, 1000, 4, 32)
    assert _call(lib, wsb=need - 1) == E_WORKSPACE
    assert str(need).encode() in lib.kd_last_error()


def _call_fwd(lib, **kw):
    base = dict(h=0x100000, W=0x200000, dtype=1, idx=0x300000, p=0x400000, mask=None, N=64,
                d=64, V=1000, K=4, chunk=32, loss=0x500000, row_lse=0x900000, row_loss=None,
                zg=None, ws=0x800000, wsb=1 << 40, stream=None)
    base.update(kw)
    b = base
    return lib.kd_chunked_kl_fwd(b["h"], b["W"], b["dtype"], b["idx"], b["p"], b["mask"],
                                 b["N"], b["d"], b["V"], b["K"], b["chunk"], b["loss"],
                                 b["row_lse"], b["row_loss"], b["zg"], b["ws"], b["wsb"],
                                 b["stream"])


def _call_bwd(lib, **kw):
    base = dict(h=0x100000, W=0x200000, dtype=1, idx=0x300000, p=0x400000, mask=None, N=64,
                d=64, V=1000, K=4, chunk=32, row_lse=0x900000, g=0xA00000, dh=0x600000,
                dW=0x700000, ws=0x800000, wsb=1 << 40, stream=None)
    base.update(kw)
    b = base
    return lib.kd_chunked_kl_bwd(b["h"], b["W"], b["dtype"], b["idx"], b["p"], b["mask"],
                                 b["N"], b["d"], b["V"], b["K"], b["chunk"], b["row_lse"],
                                 b["g"], b["dh"], b["dW"], b["ws"], b["wsb"], b["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(loss=None), E_ARG),
    (dict(row_lse=None), E_ARG),     # the state the backward reads is required
    (dict(W=None), E_ARG),
    (dict(h=None), E_ARG),
    (dict(row_lse=0x900002), E_ARG),
    (dict(h=0x100008), E_ARG),
    (dict(d=60), E_UNSUPPORTED),
    (dict(wsb=1000), E_WORKSPACE),
])
def test_forward_entry_rejects_bad_calls_on_host(lib, kw, code):
    assert _call_fwd(lib, **kw) == code
    assert lib.kd_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(row_lse=None), E_ARG),
    (dict(g=None), E_ARG),
    (dict(dh=None), E_ARG),
    (dict(dW=None), E_ARG),
    (dict(g=0xA00002), E_ARG),
    (dict(dW=0x700004), E_ARG),
    (dict(d=60), E_UNSUPPORTED),
    (dict(K=0), E_ARG),
    (dict(wsb=1000), E_WORKSPACE),
])
def test_backward_entry_rejects_bad_calls_on_host(lib, kw, code):
    assert _call_bwd(lib, **kw) == code
    assert lib.kd_last_error()


def _call_topk(lib, **kw):
    base = dict(logits=0x100000, dtype=1, N=64, V=1000, K=100, idx=0x200000, p=0x300000,
                lse=None, ws=0x400000, wsb=256, stream=None)
    base.update(kw)
    b = base
    return lib.kd_teacher_topk(b["logits"], b["dtype"], b["N"], b["V"], b["K"], b["idx"], b["p"],
                               b["lse"], b["ws"], b["wsb"], b["stream"])


def test_topk_workspace_query(lib):
    out = ctypes.c_size_t(0)
    assert lib.kd_topk_workspace_bytes(ctypes.byref(out)) == OK and out.value == 256


@pytest.mark.parametrize("kw,code", [
    (dict(K=1001), E_ARG),            # K > V
    (dict(K=0), E_ARG),
    (dict(K=257), E_UNSUPPORTED),     # above the largest supported K
    (dict(V=0), E_ARG),
    (dict(N=-1), E_ARG),
    (dict(dtype=5), E_ARG),
    (dict(logits=None), E_ARG),
    (dict(idx=None), E_ARG),
    (dict(logits=0x100001), E_ARG),   # bf16 logits must be 2-byte aligned
    (dict(p=0x300002), E_ARG),
    (dict(ws=None), E_ARG),
    (dict(ws=0x400010), E_ARG),
    (dict(wsb=100), E_WORKSPACE),
    (dict(V=1 << 29, K=10), E_UNSUPPORTED),
])
def test_topk_rejects_bad_calls_on_host(lib, kw, code):
    assert _call_topk(lib, **kw) == code
    assert lib.kd_last_error()


def test_topk_with_no_rows_does_nothing(lib):
    assert _call_topk(lib, N=0, logits=None, idx=None, p=None) == OK


def _call_shard_fwd(lib, **kw):
    base = dict(h=0x100000, W=0x200000, dtype=1, idx=0x300000, p=0x400000, N=64, d=64, Vs=500,
                v0=500, Vt=1000, K=4, chunk=32, m=0x500000, s=0x600000, pz=0x700000, zg=None,
                ws=0x800000, wsb=1 << 40, stream=None)
    base.update(kw)
    b = base
    return lib.kd_vocab_shard_fwd(b["h"], b["W"], b["dtype"], b["idx"], b["p"], b["N"], b["d"],
                                  b["Vs"], b["v0"], b["Vt"], b["K"], b["chunk"], b["m"], b["s"],
                                  b["pz"], b["zg"], b["ws"], b["wsb"], b["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(v0=600), E_ARG),            # shard runs past the vocabulary
    (dict(v0=-1), E_ARG),
    (dict(Vt=400), E_ARG),            # vocabulary smaller than the shard
    (dict(m=None), E_ARG),            # statistics outputs are required
    (dict(Vt=1 << 25, v0=0), E_ARG),  # vocabulary above 2^24
])
def test_shard_forward_rejects_bad_shards_on_host(lib, kw, code):
    assert _call_shard_fwd(lib, **kw) == code
    assert lib.kd_last_error()


def _call_f32dh(lib, **kw):
    base = dict(h=0x100000, W=0x200000, dtype=1, idx=0x300000, p=0x400000, mask=None, N=64,
                d=64, V=1000, K=4, chunk=32, loss=0x500000, dh=0x600000, dW=0x700000,
                row_loss=None, row_lse=None, zg=None, ws=0x800000, wsb=1 << 40, stream=None)
    base.update(kw)
    b = base
    return lib.kd_chunked_kl_fwd_bwd_f32dh(
        b["h"], b["W"], b["dtype"], b["idx"], b["p"], b["mask"], b["N"], b["d"], b["V"],
        b["K"], b["chunk"], b["loss"], b["dh"], b["dW"], b["row_loss"], b["row_lse"], b["zg"],
        b["ws"], b["wsb"], b["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dh=None), E_ARG),
    (dict(dh=0x600004), E_ARG),      # float32 dh still 16-byte aligned
    (dict(loss=None), E_ARG),
    (dict(d=60), E_UNSUPPORTED),
    (dict(wsb=1000), E_WORKSPACE),
])
def test_float32_dh_entry_rejects_bad_calls_on_host(lib, kw, code):
    assert _call_f32dh(lib, **kw) == code
    assert lib.kd_last_error()


def _call_scale(lib, **kw):
    base = dict(g=0x100000, dh32=0x200000, dh=0x300000, dtype=1, N=64, d=64, dW=0x400000,
                V=1000, stream=None)
    base.update(kw)
    b = base
    return lib.kd_scale_grads(b["g"], b["dh32"], b["dh"], b["dtype"], b["N"], b["d"], b["dW"],
                              b["V"], b["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), E_ARG),
    (dict(dh32=None), E_ARG),
    (dict(dh=None), E_ARG),
    (dict(dW=None), E_ARG),
    (dict(dtype=5), E_ARG),
    (dict(N=-1), E_ARG),
    (dict(d=0), E_ARG),
    (dict(dh32=0x200008), E_ARG),    # not 16-byte aligned
    (dict(dW=0x400004), E_ARG),
    (dict(g=0x100002), E_ARG),
])
def test_scale_grads_rejects_bad_calls_on_host(lib, kw, code):
    assert _call_scale(lib, **kw) == code
    assert lib.kd_last_error()


def test_scale_grads_with_nothing_to_scale_does_nothing(lib):
    assert _call_scale(lib, N=0, V=0, dh32=None, dh=None, dW=None) == OK


def test_clock_stamp_rejects_bad_arguments_before_any_gpu_work(lib):
    """kd_clock_stamp and kd_wall_clock_khz check their arguments on the host first, so
    these calls return KD_E_ARG without touching a device (none is needed here)."""
    assert lib.kd_clock_stamp(None, 8, None) == E_ARG
    assert lib.kd_last_error()
    assert lib.kd_clock_stamp(0x1004, 8, None) == E_ARG          # not 8-byte aligned
    assert lib.kd_clock_stamp(0x1000, 0, None) == E_ARG
    assert lib.kd_clock_stamp(0x1000, 65537, None) == E_ARG
    assert lib.kd_wall_clock_khz(None) == E_ARG


def test_async_call_requires_an_aligned_status_before_any_gpu_work(lib):
    """kd_chunked_kl_fwd_bwd_async checks its status pointer on the host first: a missing
    or misaligned one returns KD_E_ARG without touching a device."""
    args = [0x1000, 0x2000, 1, 0x3000, 0x4000, None, 64, 64, 100, 4, 32,
            0x5000, 0x6000, 0x7000, None, None, None]
    assert lib.kd_chunked_kl_fwd_bwd_async(*args, None, 0x8000, 1 << 20, None) == E_ARG
    assert lib.kd_last_error()
    assert lib.kd_chunked_kl_fwd_bwd_async(*args, 0x9002, 0x8000, 1 << 20, None) == E_ARG
