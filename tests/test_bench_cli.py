"""bench.py's command line on the host: several GPUs are refused with a
message before anything touches a GPU (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_several_gpus_are_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_a_multi_rank_launch_is_refused():
    r = run_bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode != 0
    assert "WORLD_SIZE 4" in (r.stdout + r.stderr)
