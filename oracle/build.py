"""Compile the C oracle (attn_oracle.c) into oracle/_build/liboracle.so with gcc.

Test infrastructure only: see the header of attn_oracle.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    # Plain -O2, no -ffast-math and no -march: the oracle keeps the C
    # evaluation order and IEEE double rounding.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lpthread", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
