"""Compile oracle/tq_loops.c into oracle/_tq_loops.so with gcc (test
infrastructure only).  Runs nothing of the oracle itself: it only builds the
loop library the oracle loads."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_loops.c")
LIB = os.path.join(HERE, "_tq_loops.so")


def build(force: bool = False) -> str:
    """Build the library when forced, missing or older than its source; return its path."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
