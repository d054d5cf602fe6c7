"""bench.py's command line on the host: it measures one GPU only, so asking
for more GPUs (or starting it under a multi-process launcher) exits with a
message and status 2 before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run(["--gpus", "2"])
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr


def test_multi_process_launch_is_refused():
    r = run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
