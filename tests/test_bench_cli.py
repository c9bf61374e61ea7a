"""bench.py's command line on the host: more than one GPU is refused with a
message, before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line
