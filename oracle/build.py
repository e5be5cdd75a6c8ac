"""Builds the oracle's C folds: ``gcc`` -> ``oracle/_fold.so``.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "fold.c")
    out = os.path.join(HERE, "_fold.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-Werror", "-shared", "-fPIC", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
