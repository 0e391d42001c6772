"""Build the HIP library ``libpaged_attn.so`` for gfx950, in-tree.

    python -m paged_gqa_attention_02_amd.build

Every kernel is compiled with packed-fp32 VALU instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpaged_attn.so")
SOURCES = ["api.cpp", "decode.hip", "merge.hip", "gather.hip", "extend.hip", "append.hip",
           "mla.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    return res.returncode, err


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object in parallel (one hipcc each), then
    link the shared library; the library is replaced only when all succeed."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC] + flags() + ["-c", "-o", o, s] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
        if err and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([HIPCC] + flags() + ["-shared", "-o", tmp] + objs + ["-ldl"])
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
