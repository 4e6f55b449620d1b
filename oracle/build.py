"""Compile the C oracle into oracle/libsgc_oracle.so (test infrastructure).

The oracle is plain C built with gcc; -ffp-contract=off keeps every fp32
operation a separately rounded IEEE operation (x86-64 SSE arithmetic).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sgc_oracle.c")
LIB = os.path.join(HERE, "libsgc_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
