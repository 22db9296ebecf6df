"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math, no floating-point contraction: every fp32/fp64
operation in the oracle rounds exactly where its source says it does.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fgb_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force=True):
    """Compile oracle/fgb_oracle.c into oracle/liboracle.so."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
