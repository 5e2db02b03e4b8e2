"""bench.py's command line on the CPU: it measures one GPU only, so any
request for more (a --gpus count above 1, or a launcher's WORLD_SIZE) ends
with a message and status 2 before anything touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env_extra", [(["--gpus", "2"], None),
                                            (["--gpus", "8", "--steps", "5"], None),
                                            ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env_extra):
    r = _run(args, env_extra)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
