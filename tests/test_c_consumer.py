"""The C ABI from plain C: tests/c_consumer/mla_c_consumer.c includes
include/mla_decode.h alone and links libmla_decode.so (no Python, no torch)."""

import os
import shutil
import subprocess

import pytest

from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_consumer", "mla_c_consumer.c")
PKG = os.path.join(ROOT, "latent_attention_decode_amd")
ROCM = "/opt/rocm"


def _build(tmp_path, gpu: bool) -> str:
    exe = str(tmp_path / ("mla_c_gpu" if gpu else "mla_c_host"))
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), SRC,
           "-L", PKG, "-lmla_decode", f"-Wl,-rpath,{PKG}", "-o", exe]
    if gpu:
        cmd[1:1] = ["-DMLA_C_CONSUMER_GPU", "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include"]
        cmd += ["-L", f"{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    else:
        cmd.insert(1, "-pedantic")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_caller_host_paths(tmp_path):
    r = subprocess.run([_build(tmp_path, False), "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
def test_c_caller_decodes_closed_forms(tmp_path):
    r = subprocess.run([_build(tmp_path, True), "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr
