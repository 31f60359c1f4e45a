"""Compile the gfx950 library in-tree with hipcc: liba2av.so (release) and
liba2av_debug.so (the same sources with -DA2AV_DEBUG=1: device-side bounds checks on
every row index and table value the kernels turn into an address, failures reported as
status bit A2AV_ST_BOUNDS).  The two compile side by side.

Flags: -O3 for gfx950 only; packed-FP32 instruction selection switched off (the
kernels' float code is scalar FMA); no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liba2av.so")
DEBUG_LIB = os.path.join(HERE, "liba2av_debug.so")
SOURCES = ["a2av_api.hip", "a2av_kernels.hip", "a2av_measure.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    """Builds both libraries (in parallel); returns the release library's path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = []
    for out, extra in ((LIB, []), (DEBUG_LIB, ["-DA2AV_DEBUG=1"])):
        cmd = [HIPCC] + FLAGS + extra + ["-o", out + ".tmp"] + srcs
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, cmd, subprocess.Popen(cmd)))
    failed = [cmd for _, cmd, p in jobs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    for out, _, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


def device_asm(out_dir: str) -> list:
    """Write the gfx950 assembly of every source into out_dir (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for s in SOURCES:
        o = os.path.join(out_dir, s.replace(".hip", f"-{ARCH}.s"))
        cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] + \
              ["--offload-device-only", "-S", "-o", o, os.path.join(CSRC, s)]
        subprocess.run(cmd, check=True)
        outs.append(o)
    return outs


if __name__ == "__main__":
    print(build(verbose=True))
