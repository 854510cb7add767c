"""bench.py's command-line contract, checked without a GPU: one GPU only
(more exits with a message and status 2), and the workloads it offers."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_workloads_listed():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("phi_layer", "qwen_chunk", "ds_draft", "draft_formats", "qwen_rounds",
              "route_fidelity"):
        assert w in r.stdout, w
