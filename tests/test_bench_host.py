"""bench.py's refusal of more than one GPU, checked before it touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    for extra in ([], ["--topk"], ["--memory-sweep"]):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", *extra],
                             capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert res.returncode == 2, (extra, res.returncode, res.stderr[-500:])
        assert "one GPU only" in res.stderr and res.stdout == ""
