"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

The C oracle is rebuilt with gcc's sanitizers, and the library's host code (the
C ABI: validation, the plan, argument checks) with the HIP compiler's host-side
sanitizers, each into a temporary directory. The oracle pins and the CPU tests
of the library then run against those builds in a child Python process with
the matching sanitizer runtime preloaded; any report ends that process with a
nonzero status. No GPU code is built with a sanitizer and nothing reaches a
kernel launch."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_05_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(bootstrap, preload, tmp_path):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    log = tmp_path / "child.log"
    with open(log, "w") as f:
        rc = subprocess.call([sys.executable, "-c", bootstrap], cwd=ROOT, env=env, stdout=f,
                             stderr=subprocess.STDOUT, timeout=600)
    text = log.read_text()
    assert rc == 0 and "runtime error" not in text and "ERROR: AddressSanitizer" not in text, \
        text[-4000:]


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", str(lib),
                           os.path.join(ROOT, "oracle", "decode_oracle.c"), "-lm"])
    preload = ":".join(subprocess.check_output(["gcc", f"-print-file-name={n}"]).decode().strip()
                       for n in ("libasan.so", "libubsan.so"))
    bootstrap = (
        "import sys, oracle, pytest\n"
        f"oracle._LIB = {str(lib)!r}\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        "    'tests/test_oracle.py', 'tests/test_ragged_oracle.py', 'tests/test_tokens_oracle.py']))\n")
    run_child(bootstrap, preload, tmp_path)


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not runtimes:
        pytest.skip("the HIP compiler or its sanitizer runtime is not installed")
    from decode_attention_05_amd import build as B
    objs = [os.path.join(B.HERE, "_build", src + ".o") for src in B.SOURCES if src.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api = tmp_path / "api_san.o"
    lib = tmp_path / "libdecode_attn_san.so"
    # host code only: every sanitizer flag is scoped to the host compilation
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.check_call([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
                           "-fno-omit-frame-pointer", *host_san, "-I", os.path.join(ROOT, "include"),
                           "-c", os.path.join(CSRC, "api.cpp"), "-o", str(api)],
                          stderr=subprocess.DEVNULL)
    subprocess.check_call([hipcc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-shared-libsan", "-o", str(lib), str(api), *objs])
    bootstrap = (
        "import sys, pytest\n"
        "import decode_attention_05_amd as da\n"
        f"da.library_path = {str(lib)!r}\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        "    'tests/test_library_cpu.py']))\n")
    run_child(bootstrap, runtimes[-1], tmp_path)
