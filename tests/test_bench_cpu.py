"""bench.py's command-line contract, checked without a GPU: one GPU only (every
tensor-parallel rank is emulated on one device), and no CPU stand-in when the
GPU is missing: it exits with a message and prints no result line."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(args, env)
    assert r.returncode != 0
    assert "not supported" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the run without a GPU")
def test_no_gpu_no_result_line():
    r = run_bench(["--steps", "1", "--warmup", "0"])
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""
