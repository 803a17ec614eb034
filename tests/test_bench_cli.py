"""The bench's command-line contract, checked without a GPU: a request for
more than one GPU (by flag or by a launcher's WORLD_SIZE) exits with status
2 and says why before anything touches a device, and --help lists the
workloads, the headline first."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          env=dict(os.environ, **(env or {})), timeout=120)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], None), (["--gpus", "8"], None),
                      ([], {"WORLD_SIZE": "2"})):
        out = _run(args, env)
        assert out.returncode == 2, (args, env, out.stdout, out.stderr)
        assert "measures one GPU" in out.stderr
        assert out.stdout == ""


def test_help_lists_the_workloads():
    out = _run(["--help"])
    assert out.returncode == 0
    for w in ("headline", "llama3-8b", "gpt2-small", "moe-16l", "ring-1gib",
              "llama3-8b-ipg", "share-1b", "llama3-8b-placement"):
        assert w in out.stdout


def test_placement_needs_a_set_and_a_call():
    for args in (["--sets", "0"], ["--calls", "0"]):
        out = _run(["--workload", "llama3-8b-placement", *args])
        assert out.returncode == 2, (args, out.stdout, out.stderr)
        assert "at least 1" in out.stderr
        assert out.stdout == ""
