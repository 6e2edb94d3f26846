"""Build the plain-C consumers of the C ABI (consumer.c: host-side calls; consumer_gpu.c: one rank share on the
GPU) with gcc against include/ and the in-tree libcpthd.so, into tests/c_abi/bin/.

    python tests/c_abi/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBDIR = os.path.join(ROOT, "context_causal_thd_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "bin")
PROGRAMS = ("consumer", "consumer_gpu")


def command(name, out):
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), os.path.join(HERE, name + ".c"),
            "-L", LIBDIR, "-lcpthd", f"-Wl,-rpath,{LIBDIR}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out]


def build(out_dir=BIN):
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for name in PROGRAMS:
        out = os.path.join(out_dir, name)
        r = subprocess.run(command(name, out), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"gcc failed for {name}.c:\n{r.stdout}")
        outs.append(out)
    return outs


if __name__ == "__main__":
    print("\n".join(build(*sys.argv[1:])))
