"""Compile the oracle's C code into ``oracle/_oracle.so`` with gcc (test infrastructure)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "combine.c")
LIB = os.path.join(HERE, "_oracle.so")
THREADS_SRC = os.path.join(HERE, "protocol_threads.c")
THREADS_EXE = os.path.join(HERE, "_protocol_threads")


def _compile(cmd, out, verbose):
    tmp = out + f".tmp{os.getpid()}"
    cmd = cmd + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """The combine oracle library and the threaded protocol executor."""
    _compile(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", SRC], LIB, verbose)
    _compile(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", THREADS_SRC, "-lpthread"], THREADS_EXE, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
