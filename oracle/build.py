"""Build step for the fp64 CPU oracle (plain C, gcc) -- test infrastructure."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libkda_oracle.so")


def build_oracle(cc: str = "gcc", verbose: bool = False) -> str:
    """Compile kda_oracle.c into oracle/libkda_oracle.so (always rebuilds).

    No -ffast-math: the oracle keeps IEEE fp64 semantics and its summation
    order."""
    src = os.path.join(_HERE, "kda_oracle.c")
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
