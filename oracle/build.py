"""Compile the CPU oracle (test infrastructure) into oracle/libmxq_oracle.so.

Plain gcc, no vector intrinsics, no fast-math and no floating-point
contraction, so each operation in mxq_oracle.c is one IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmxq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        os.path.join(HERE, "mxq_oracle.c"),
        "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
