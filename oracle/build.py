"""Compile the fp64 C oracle into ``oracle/_diffattn_oracle.so``.

Test infrastructure: the compiled oracle is used only by the tests, the smoke
check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "diffattn_oracle.c")
LIB = os.path.join(HERE, "_diffattn_oracle.so")

# -ffp-contract=off: no fused multiply-add contraction, so every product and
# sum is rounded as written; no -ffast-math, so sums keep their index order.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
