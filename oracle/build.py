"""Build the CPU oracle (test infrastructure only).

Compiles oracle/dspark_oracle.cpp into oracle/libdspark_oracle.so with the
host C++ compiler.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dspark_oracle.cpp")
LIB = os.path.join(HERE, "libdspark_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle library (always) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-shared", "-fPIC",
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
