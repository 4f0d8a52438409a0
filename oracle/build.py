"""Build liboracle.so, the plain sequential C oracle (test infrastructure only).

-ffp-contract=off: no multiply-add contraction; -fno-fast-math: IEEE semantics;
x86-64 SSE2 scalar arithmetic with the default MXCSR (round to nearest even,
gradual underflow; the oracle flushes subnormals explicitly).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fopenmp", "-fPIC", "-shared",
           os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
