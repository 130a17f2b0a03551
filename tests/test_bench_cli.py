"""bench.py's command line on the host: it runs on one GPU only and says so for --gpus N > 1 (or a
multi-rank launch), before touching any device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for args, extra in ((["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None), ([], {"WORLD_SIZE": "2"})):
        res = _run(args, extra)
        assert res.returncode == 2, (args, res.stdout, res.stderr)
        line = json.loads(res.stdout.strip().splitlines()[-1])
        assert "one GPU" in line["error"]
