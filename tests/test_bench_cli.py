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


def test_rotation_bounds():
    """Copies the timed loop rotates through: >= 512 MB between reuses for the big
    workloads, at least 4 for one layer, at most 128 for cache-sized ones."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.rotation(152e6, 1) == 4        # the 32-sequence workload
    assert bench.rotation(404e6, 48) == 1       # 48 layers already exceed the cache
    assert bench.rotation(4.3e6, 1) == 120      # one sequence of 16 nodes
    assert bench.rotation(7e3, 1) == 128        # the tiny tree: capped
    for per_copy in (1e3, 1e6, 5e6, 1e8, 1e9):
        r = bench.rotation(per_copy, 1)
        assert 4 <= r <= 128 and (r == 128 or r * per_copy >= 512e6 or r == 4)


def test_fused_schedule_takes_the_fused_kernels_workloads():
    """--schedule fused is offered for the workloads the fused kernel runs (bf16, head
    dim 64 or 128, trees of at most 32 nodes): the batched, chain and 23-node tree
    workloads, not the 65-node stress trees or the fp32 tiny tree."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    assert [bench.fused_supported(W.get_config(n)) for n in ("tiny", "chain", "ddtree22", "batched", "stress")] == \
        [False, True, True, True, False]
    old = sys.argv
    try:
        sys.argv = ["bench.py", "--schedule", "fused"]
        assert bench.parse().schedule == "fused"
        sys.argv = ["bench.py"]
        assert bench.parse().schedule == "separate"
    finally:
        sys.argv = old
