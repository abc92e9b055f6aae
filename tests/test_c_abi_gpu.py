"""The library called from C, with no Python or PyTorch in the caller's process
(tests/c_abi/kd_driver.c: buffers from hipMalloc, a stream of its own): the one-call
loss with its per-row outputs, and the forward and backward halves, against the oracle
on the same seeded inputs; and an invalid teacher index refused with KD_E_INDEX, a
message, and the outputs untouched.  The boundary is the C ABI of include/kdkl.h
(codewithpapers.app record: the loss's arguments h, W, teacher indices and
probabilities, mask and chunk)."""
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, ZG_TOL, grad_err, max_abs_rel, rel

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "kd_driver")
KD_E_INDEX = 2


def _write_problem(path, inp):
    cfg = inp.cfg
    dt = 1 if cfg.dtype == "bf16" else 0
    with open(path, "wb") as f:
        f.write(struct.pack("<7q", 0x4C4B444B, dt, cfg.N, cfg.d, cfg.V, cfg.K, cfg.chunk))
        for a, t in ((inp.h, None), (inp.W, None), (inp.idx, np.int32), (inp.p, np.float32),
                     (inp.mask, np.uint8)):
            f.write(np.ascontiguousarray(a if t is None else a.astype(t)).tobytes())


def _read_outputs(path, inp):
    cfg = inp.cfg
    N, d, V, K = cfg.N, cfg.d, cfg.V, cfg.K
    raw = open(path, "rb").read()
    pos = 0

    def take(n, dtype):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    def take_h(n):
        if cfg.dtype == "bf16":
            return synth.bf16_bits_to_f32(take(n, np.uint16)).astype(np.float64)
        return take(n, np.float32).astype(np.float64)

    out = dict(loss=float(take(1, np.float32)[0]), dh=take_h(N * d).reshape(N, d),
               dW=take(V * d, np.float32).astype(np.float64).reshape(V, d),
               row_loss=take(N, np.float32).astype(np.float64),
               row_lse=take(N, np.float32).astype(np.float64),
               zg=take(N * K, np.float32).astype(np.float64).reshape(N, K),
               loss2=float(take(1, np.float32)[0]), dh2=take_h(N * d).reshape(N, d),
               dW2=take(V * d, np.float32).astype(np.float64).reshape(V, d))
    out["rc_bad"], out["described"], out["untouched"] = (int(x) for x in take(3, np.int32))
    assert pos == len(raw), (pos, len(raw))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_c_caller_against_the_oracle(tmp_path, dtype):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built (run __graft_entry__.build())")
    inp = synth.make(1, seed=91, N=700, d=264, V=3001, K=7, chunk=300, dtype=dtype)
    inp.mask[[0, 299, 699]] = 0
    inp.idx[5, 1] = inp.idx[5, 0]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_problem(src, inp)
    print(f"kd_driver {dtype} N={inp.cfg.N} d={inp.cfg.d} V={inp.cfg.V}", flush=True)
    res = subprocess.run([DRIVER, str(src), str(dst)], capture_output=True, text=True,
                         timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    got = _read_outputs(dst, inp)
    ref = oracle.forward_backward(inp.h64(), inp.W64(), inp.idx, inp.p, inp.mask)
    tol = TOL[dtype]
    errs = dict(loss=rel(got["loss"], ref["loss"]), dh=grad_err(dtype, got["dh"], ref["dh"]),
                dW=grad_err(dtype, got["dW"], ref["dW"]),
                row_lse=max_abs_rel(got["row_lse"], ref["row_lse"]),
                row_loss=max_abs_rel(got["row_loss"], ref["row_loss"]),
                zg=max_abs_rel(got["zg"], ref["zg"]),
                split_loss=rel(got["loss2"], ref["loss"]),
                split_dh=grad_err(dtype, got["dh2"], ref["dh"]),
                split_dW=grad_err(dtype, got["dW2"], ref["dW"]))
    print(dtype, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k in ("loss", "split_loss", "row_lse"):
        assert errs[k] <= tol["loss"], errs
    assert errs["row_loss"] <= 10 * tol["loss"], errs
    for k in ("dh", "dW", "split_dh", "split_dW"):
        assert errs[k] <= tol["grad"], errs
    assert errs["zg"] <= ZG_TOL, errs
    assert np.all(got["dh"][inp.mask == 0] == 0.0) and np.all(got["dh2"][inp.mask == 0] == 0.0)
    # the bad index: refused after validation, described, nothing written
    assert got["rc_bad"] == KD_E_INDEX and got["described"] == 1 and got["untouched"] == 1
