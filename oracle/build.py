"""Build the CPU oracle (test infrastructure) into oracle/liborc.so.

Flags keep every float operation a single IEEE binary32 operation rounded to
nearest even: no contraction into FMA, no fast-math, no target-specific ISA.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liborc.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-pthread", os.path.join(HERE, "echo_oracle.c"),
           os.path.join(HERE, "echo_oracle_mt.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
