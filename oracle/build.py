"""Build the CPU oracle (plain C11, gcc -O2, no fast-math) into oracle/liba2av_oracle.so.

Test infrastructure only: the oracle is loaded by tests/, by the smoke check and by the
cpu_baseline leg of bench.py, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "a2av_oracle.c")
LIB = os.path.join(HERE, "liba2av_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
