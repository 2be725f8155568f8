"""bench.py's command line, on the CPU: the default timed-step counts per
workload and the one-GPU guard (no device work)."""
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def _args(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


@pytest.mark.parametrize("config,steps", [
    ("long_context", 100),         # one layer of 32,768-token sequences: 100 tokens are 0.3% more bytes
    ("long_context_fp8", 100),
    ("full_step", 20),             # 32 layers, sequences of about 500 tokens grow by one per step
    ("full_step_fp8", 20),
    ("single_layer", 20),          # short sequences: the pool holds a few dozen steps' growth
    ("shared_prefix", 20),
    ("tiny", 20),
    ("prefill_prompts", 20),
    ("prefill_chunked", 20),
    ("prefill_prompts_fp8", 20),
    ("prefill_chunked_fp8", 20),
])
def test_default_steps_per_workload(config, steps):
    wl = workloads.CONFIGS[config]()
    assert bench.with_steps(_args("--config", config), wl).steps == steps


def test_given_steps_win():
    wl = workloads.CONFIGS["long_context"]()
    assert bench.with_steps(_args("--steps", "7"), wl).steps == 7


def test_with_steps_leaves_the_given_args_alone():
    a = _args()
    bench.with_steps(a, workloads.CONFIGS["long_context"]())
    assert a.steps is None            # the 32-layer leg resolves its own default from these


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_outlasts_a_small_pool():
    """The oracle's timing leg keeps stepping a batch whose pool fills up: the
    tiny batch's 32 blocks hold about a hundred steps of growth, and the leg
    starts again from the set-up state instead of failing."""
    r = bench.cpu_baseline("tiny", 1.0)
    steps = int(r["sample"].split(";")[1].split()[0])
    assert steps > 150, r["sample"]
    assert r["value"] > 0 and r["kind"] == "oracle"
