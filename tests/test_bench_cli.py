"""bench.py measures one GPU: asked for more (by flag or by a distributed
launcher's WORLD_SIZE) it exits with status 2 and a message, printing no
result line.  Runs on the CPU: the check comes before any GPU work."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          cwd=ROOT, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})],
                         ids=["gpus2", "gpus8", "world2"])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(args, env)
    assert r.returncode == 2, (r.returncode, r.stderr[-400:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
