"""Build tests/c_caller/c_caller: a plain C program (gcc, HIP runtime API only) linked
against the in-tree liba2av.so, run by tests/test_c_caller_gpu.py."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "moe_alltoallv_resident_amd")
EXE = os.path.join(HERE, "c_caller")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_caller.c"), "-o", EXE,
           "-L", PKG, "-la2av", "-Wl,-rpath," + PKG,
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())
