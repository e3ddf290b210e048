"""Build the gfx950 HIP library libdspark.so in-tree with hipcc."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdspark.so")
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the generated code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libdspark.so (always) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    env = dict(os.environ)
    env.setdefault("TMPDIR", "/tmp")
    subprocess.run(cmd, check=True, env=env, cwd="/tmp")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
