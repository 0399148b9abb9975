"""bench.py's command-line contract that needs no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_source_digest_ignores_comments_only():
    sys.path.insert(0, ROOT)
    import bench
    for kernel in bench.KERNEL_SOURCES:
        d = bench.kernel_source_digest(kernel)
        assert len(d) == 16 and d == bench.kernel_source_digest(kernel)
    assert bench.kernel_source_digest("persist") != bench.kernel_source_digest("accept")
