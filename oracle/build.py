"""Compile the C oracle (``specref.c``) into ``libspecref.so`` next to it with gcc.

Test infrastructure: the oracle is built from its own single source file and
links only libm.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "specref.c")
LIB = os.path.join(HERE, "libspecref.so")


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared",
                               "-fPIC", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
