"""Build the oracle library ``oracle/libngram_oracle.so`` with gcc (host only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ngram_oracle.c")
LIB = os.path.join(HERE, "libngram_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra",
           "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
