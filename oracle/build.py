"""Build the fp64 CPU oracle library (test infrastructure only).

Compiles ``pa_oracle.c`` with gcc into ``libpa_oracle.so`` next to this file.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "libpa_oracle.so")


# AddressSanitizer + UndefinedBehaviorSanitizer build: every finding aborts.
# A process loading it must preload gcc's libasan and libubsan
# (sanitizer_preload()).
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"]


def sanitizer_preload() -> str:
    """LD_PRELOAD value for a process that loads the sanitized build."""
    libs = [subprocess.run(["gcc", "-print-file-name=" + n], capture_output=True, text=True,
                           check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    return ":".join(libs)


def build(verbose: bool = False, src: str = SRC, out: str = None,
          sanitize: bool = False) -> str:
    opt = SANITIZE if sanitize else ["-O2"]
    cmd = ["gcc"] + opt + ["-std=c99", "-fPIC", "-shared", "-pthread",
                           "-Wall", "-Wextra", "-o", (out or LIB) + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace((out or LIB) + ".tmp", out or LIB)
    return out or LIB


if __name__ == "__main__":
    print(build(verbose=True))
