"""Build the oracle's shared library with gcc (plain C, no GPU code).

Test infrastructure only; run as ``python -m oracle.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def oracle_lib_path() -> str:
    return os.path.join(HERE, "libssd_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ssd_oracle.c")
    out = oracle_lib_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-pthread",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
