"""bench.py's command line, CPU only (no GPU step is ever started here).

- more than one GPU, by flag or by a launcher's WORLD_SIZE, is refused with a
  message and exit status 2 before anything is imported or allocated;
- with no GPU the default run stops with an error instead of measuring
  anything on the CPU (there is no host fallback to time).
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def _bench(*args, env_extra=None, timeout=120):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)


@pytest.mark.parametrize("args,env", [(("--gpus", "2"), None), (("--gpus", "8"), None),
                                      ((), {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    p = _bench(*args, env_extra=env)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and "no multi-GPU path" in p.stderr
    assert p.stdout == ""  # no JSON line for the driver to mistake for a result


def test_help_lists_the_workloads():
    p = _bench("--help")
    assert p.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--routing", "--cold-rows"):
        assert opt in p.stdout


def test_no_gpu_no_measurement():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the CPU-only behaviour is not observable here")
    p = _bench("--steps", "1", "--warmup", "0")
    assert p.returncode != 0
    assert "needs a GPU" in p.stderr
    assert '"metric"' not in p.stdout


def test_kernel_split_steps():
    """The timed steps that carry an event between the two hot kernels: the
    middle of each group of four, never the first step of a longer run (it
    starts from an idle device); a run of one or two steps uses its first."""
    sys.path.insert(0, str(ROOT))
    import bench
    pick = lambda n: [i for i in range(n) if bench.kernel_split_step(i, n)]
    assert pick(20) == [2, 6, 10, 14, 18]
    assert pick(1024)[:3] == [2, 6, 10] and len(pick(1024)) == 256
    assert pick(3) == [2]
    assert pick(2) == [0] and pick(1) == [0]
