"""The Python binding rejects tensors that are not on the call's GPU before it touches the
library (CPU only: the library is replaced by an object that fails on any use)."""
import os
import types

import pytest
import torch

import output_head_kl_amd as kd


class _NoLibrary:
    def __getattr__(self, name):
        raise AssertionError(f"the library was used ({name}) before the device check")


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(kd, "_LIB", _NoLibrary())


def _inputs(device):
    h = torch.zeros((8, 16), dtype=torch.bfloat16, device=device)
    W = torch.zeros((32, 16), dtype=torch.bfloat16, device=device)
    idx = torch.zeros((8, 4), dtype=torch.int32, device=device)
    p = torch.zeros((8, 4), dtype=torch.float32, device=device)
    mask = torch.ones(8, dtype=torch.uint8, device=device)
    return h, W, idx, p, mask


@pytest.mark.parametrize("device", ["cpu", "meta"])
def test_every_entry_rejects_tensors_off_the_gpu(no_library, device):
    h, W, idx, p, mask = _inputs(device)
    lse = torch.zeros(8, dtype=torch.float32, device=device)
    g = torch.ones(1, dtype=torch.float32, device=device)
    calls = [
        lambda: kd.fwd_bwd(h, W, idx, p, mask, chunk=4),
        lambda: kd.fwd_bwd(h, W, idx, p, mask, chunk=4, dh_float32=True),
        lambda: kd.fwd(h, W, idx, p, mask, chunk=4),
        lambda: kd.bwd(h, W, idx, p, lse, g, mask, chunk=4),
        lambda: kd.chunked_kl_loss(h, W, idx, p, mask, chunk=4),
        lambda: kd.chunked_kl_loss(h, W, idx, p, mask, chunk=4, mode="recompute"),
        lambda: kd.teacher_topk(torch.zeros((8, 32), dtype=torch.bfloat16, device=device), K=4),
        lambda: kd.vocab_shard_fwd(h, W, idx, p, 0, 32, chunk=4),
        lambda: kd.vocab_shard_bwd(h, W, idx, p, lse, 0, 32, g, mask, chunk=4),
        lambda: kd.vocab_shard_combine(lse.view(1, 8), lse.view(1, 8), lse.view(1, 8), p, mask),
        lambda: kd.scale_grads(g, torch.zeros((8, 16), device=device),
                               torch.zeros((32, 16), device=device)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="CUDA|on "):
            call()


def _fake(device):
    return types.SimpleNamespace(is_cuda=torch.device(device).type == "cuda",
                                 device=torch.device(device))


def test_device_check_names_the_offending_argument():
    dev = torch.device("cuda:0")
    kd._on_device(dev, h=_fake("cuda:0"), mask=None)          # same GPU: accepted
    with pytest.raises(ValueError, match="grad_loss is on cpu"):
        kd._on_device(dev, h=_fake("cuda:0"), grad_loss=_fake("cpu"))
    with pytest.raises(ValueError, match="workspace is on cuda:1"):
        kd._on_device(dev, workspace=_fake("cuda:1"))
    with pytest.raises(ValueError, match="CUDA"):
        kd._on_device(torch.device("cpu"), h=_fake("cpu"))


def test_unknown_autograd_mode_is_rejected(no_library):
    h, W, idx, p, mask = _inputs("cpu")
    with pytest.raises(ValueError, match="mode"):
        kd.chunked_kl_loss(h, W, idx, p, mask, mode="dense")


def test_c_driver_is_built_and_checks_its_input(tmp_path):
    """The C caller used by the GPU tests is built next to the library and refuses a bad
    command line or input file before it touches a GPU."""
    import subprocess
    drv = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "kd_driver")
    assert os.path.exists(drv), "build the library first (__graft_entry__.build())"
    r = subprocess.run([drv], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    bad = tmp_path / "bad.bin"
    bad.write_bytes(b"\0" * 56)
    r = subprocess.run([drv, str(bad), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "not a problem file" in r.stderr
