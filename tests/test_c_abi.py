"""The C ABI from plain C: tests/c_abi/decode_step.c includes only moe.h and
the HIP runtime header, is compiled as C99 with gcc and linked against
libmoe.so. On the CPU it must compile and link warning-free; on the GPU it
runs one decode step through both of the library's paths and checks them
against the closed form of its inputs (it prints "ok")."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_grouped_moe_amd")
SRC = os.path.join(ROOT, "tests", "c_abi", "decode_step.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libmoe.so")):
        pytest.skip("libmoe.so is not built")
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "decode_step")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}", SRC,
           f"-L{PKG}", "-lmoe", f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_caller_compiles_and_links(tmp_path):
    _compile(tmp_path)


@pytest.mark.gpu
def test_c_caller_runs_a_decode_step(tmp_path):
    # the program runs as a child process; counting devices does not
    # initialise the GPU in this one
    import torch
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    exe = _compile(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
