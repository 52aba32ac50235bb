"""The C ABI from a C11 program (gcc, no C++, no Python between): the header
compiles as C and the host-decided parts of the calls behave as documented."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "dynamic_block_sparse_amd", "lib")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libprism.so")), reason="libprism.so not built")
@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INC), reason="needs gcc and the ROCm headers")
def test_c_client_of_the_abi(tmp_path):
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", ROCM_INC, os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", LIBDIR, "-lprism",
           f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "c abi ok"
