"""Host-side checks of bench.py that need no GPU: it refuses more than one GPU before it
touches any device, and it rejects an unknown prefix-cache type."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "8", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_unknown_cache_type_is_rejected():
    r = _run("--kv", "int4")
    assert r.returncode != 0
    assert "invalid choice" in r.stderr
