"""Builds tests/c_consumer (a plain C program that uses only include/decode_attn.h,
the HIP runtime's C API and the C oracle) next to this file. Called by the
repository's build step, never by a test."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BINARY = os.path.join(HERE, "c_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = BINARY + f".tmp{os.getpid()}"
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
        os.path.join(HERE, "c_consumer.c"),
        "-L", os.path.join(ROOT, "decode_attention_05_amd"), "-ldecode_attn",
        "-L", os.path.join(ROOT, "oracle"), "-loracle",
        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../decode_attention_05_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib"),
        "-o", tmp])
    os.replace(tmp, BINARY)
    return BINARY
