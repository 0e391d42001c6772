"""Build the fp64 CPU oracle library (test infrastructure only).

Compiles ``pa_oracle.c`` with gcc into ``libpa_oracle.so`` next to this file.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "libpa_oracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = None) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", (out or LIB) + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace((out or LIB) + ".tmp", out or LIB)
    return out or LIB


if __name__ == "__main__":
    print(build(verbose=True))
