"""Host-side checks of bench.py's command-line contract (no GPU): more than
one GPU is refused with a message before anything touches a device, and the
default run is the DeepSeek-V3-shaped prefill workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    for argv in (["--gpus", "2"], ["--gpus", "8", "--steps", "1"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                           timeout=120, cwd=ROOT)
        assert r.returncode == 2, (argv, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_exits_too():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_defaults():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.gpus == 1 and a.config == "dsv3_prefill" and a.steps > 0 and a.warmup >= 0
    assert not a.unfused and not a.permute_copy
