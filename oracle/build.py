"""Build the CPU oracle library (gcc, OpenMP, float64, no fast-math).  Test infrastructure."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "v4a_oracle.c")


def library_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def is_stale() -> bool:
    lp = library_path()
    return not os.path.exists(lp) or os.path.getmtime(lp) < os.path.getmtime(SRC)


def build(sanitize: bool = False, out: str | None = None) -> str:
    """sanitize=True: an ASan + UBSan checking build (written to `out`), same arithmetic."""
    out = out or library_path()
    tmp = out + ".tmp"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"] if sanitize else []
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-Wno-unused-parameter"] + san + ["-shared", "-fPIC", SRC, "-o",
                                                              tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
