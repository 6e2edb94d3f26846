"""The C ABI from plain C: tests/c_abi/consumer.c, compiled with gcc against include/cpthd.h and
include/cpthd_timing.h and linked to the in-tree libcpthd.so, runs host-side calls (workspace sizes, status
strings, argument refusals) with no GPU and no Python in between."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "context_causal_thd_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_links_and_calls_the_library(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libcpthd.so")):
        pytest.skip("libcpthd.so not built")
    exe = str(tmp_path / "consumer")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "consumer.c"), "-L", LIBDIR, "-lcpthd", f"-Wl,-rpath,{LIBDIR}",
           "-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout
