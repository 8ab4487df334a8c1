"""bench.py's command line on the CPU: it times one GPU's share only, so a request for more
GPUs (by flag or by a launcher's WORLD_SIZE) ends with status 2 and a message before torch or
the library is loaded."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    if env_extra:
        env.update(env_extra)
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], None), (["--gpus", "8"], None), ([], {"WORLD_SIZE": "4"})):
        r = _run(args, env)
        assert r.returncode == 2, (args, env, r.stderr)
        assert "--gpus must be 1" in r.stderr
        assert r.stdout == ""
