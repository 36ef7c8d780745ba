"""Host-side checks of bench.py's command line (no GPU is touched)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_several_gpus_are_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_help_lists_the_legs():
    r = run("--help")
    assert r.returncode == 0
    for leg in ("hybrid", "cfgpair", "causal", "chunked", "stream", "copy"):
        assert leg in r.stdout
