"""The C ABI from plain C: tests/c_consumer (built by the repository's build
step) plans and runs a dense and a sparse decode through include/decode_attn.h
with raw HIP device memory, and checks them against the fp64 oracle."""

import os
import subprocess

import pytest

from tests import c_consumer_build

pytestmark = pytest.mark.gpu


def test_c_consumer():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(c_consumer_build.BINARY):
        pytest.fail("tests/c_consumer is not built; run __graft_entry__.build() first")
    r = subprocess.run([c_consumer_build.BINARY], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer ok" in r.stdout
