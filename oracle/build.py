"""Build liboracle.so from kvt_oracle.c with the host C compiler (no HIP, no GPU code).

Test infrastructure only: the oracle is compiled so it can check the library, never to serve it.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "kvt_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
