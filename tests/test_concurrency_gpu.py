"""Calls from two host threads at once, each with its own stream, workspace and outputs:
the library keeps no device state between calls and its only host state (the last
error) is per thread, so every result equals the same call made alone, bit for bit
(the calls are deterministic)."""
import threading

import pytest

import synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def test_two_threads_on_two_streams_match_the_calls_made_alone(torch_cuda):
    import output_head_kl_amd as kd
    torch = torch_cuda
    inps = [synth.make(1, seed=s, N=1500, d=264, V=3001, K=7, chunk=300) for s in (41, 42)]
    dev = [to_device(inp, torch) for inp in inps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()

    def one(i, workspace):
        h, W, idx, p, mask = dev[i]
        with torch.cuda.stream(streams[i]):
            if i == 0:
                out = kd.fwd_bwd(h, W, idx, p, mask, chunk=300, rows=True,
                                 workspace=workspace, stream=streams[i])
            else:  # the second thread runs the split pair
                loss, lse = kd.fwd(h, W, idx, p, mask, chunk=300, workspace=workspace,
                                   stream=streams[i])
                dh, dW = kd.bwd(h, W, idx, p, lse, None, mask, chunk=300, workspace=workspace,
                                stream=streams[i])
                out = (loss, lse, dh, dW)
            out = [t.clone() for t in out]
            streams[i].synchronize()
            return out

    def workspace(i):
        inp = inps[i]
        with torch.cuda.stream(streams[i]):
            return torch.empty(kd.workspace_bytes(inp.cfg.N, inp.cfg.d, inp.cfg.V, inp.cfg.K,
                                                  300), dtype=torch.uint8, device="cuda")

    alone = [one(i, workspace(i)) for i in range(2)]
    got, errors = [[], []], []

    def run(i):
        try:
            ws = workspace(i)
            for _ in range(4):
                got[i].append(one(i, ws))
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=180)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i in range(2):
        assert len(got[i]) == 4
        for outs in got[i]:
            for a, b in zip(outs, alone[i]):
                assert torch.equal(a, b)
