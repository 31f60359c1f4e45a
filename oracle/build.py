"""Build the CPU oracle (plain C11, gcc -O2, no fast-math) into oracle/liba2av_oracle.so.

Test infrastructure only: the oracle is loaded by tests/, by the smoke check and by the
cpu_baseline leg of bench.py, never by the product path.

`build(sanitize=True)` builds the same source with AddressSanitizer and
UndefinedBehaviorSanitizer (every finding fatal) into oracle/liba2av_oracle_san.so,
which the oracle package loads instead when A2AV_ORACLE_SANITIZED=1 is set; the process
must then have the sanitizer runtime preloaded (see `sanitizer_runtime`).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "a2av_oracle.c")
LIB = os.path.join(HERE, "liba2av_oracle.so")
LIB_SANITIZED = os.path.join(HERE, "liba2av_oracle_san.so")

_COMMON = ["gcc", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra"]
_SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = LIB_SANITIZED if sanitize else LIB
    cmd = _COMMON + (_SANITIZE if sanitize else ["-O2"]) + ["-o", lib + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of gcc's AddressSanitizer runtime, to preload into a process that loads the
    sanitized oracle."""
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True, text=True)
    return out.stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
