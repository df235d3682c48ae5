"""Host-side behaviour of bench.py that needs no GPU.

The benchmark measures one GPU: asked for more it must refuse with a message
and a non-zero status, and on a machine without a GPU it must fail loudly
instead of measuring anything else (there is no CPU fallback of the hot path).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT, env=e)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert "{" not in r.stdout   # no JSON line


def test_several_ranks_are_refused():
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode != 0
    assert "{" not in r.stdout


def test_no_gpu_fails_loudly():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _bench("--steps", "2", "--warmup", "1")
    assert r.returncode != 0
    assert "GPU" in (r.stdout + r.stderr)
    assert "{" not in r.stdout
